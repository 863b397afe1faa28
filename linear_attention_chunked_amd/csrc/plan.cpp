// Host-side scheduler (see plan.hpp).  Plain C++: no HIP calls, so the
// argument checks and plans can be exercised without a GPU.
#include "plan.hpp"

#include <stdlib.h>

#include <algorithm>
#include <cstdio>
#include <numeric>

namespace gdr {

bool parse_problem(int B, int64_t T, int H, int DK, int DV, int N, const int32_t* cu, int dtype,
                   int state_layout, const int32_t* pool_idx, int pool_size, Problem& p, std::string& err) {
  if (B < 1 || T < 0 || H < 1) {
    err = "B >= 1, T >= 0 and H >= 1 are required";
    return false;
  }
  auto dim_ok = [](int d) { return d == 64 || d == 128 || d == 256; };
  if (!(dim_ok(DK) && dim_ok(DV))) {
    err = "DK and DV must each be 64, 128 or 256";
    return false;
  }
  if (dtype == 0 && (DK == 256 || DV == 256)) {
    err = "DK or DV = 256 is supported for bfloat16 storage only";
    return false;
  }
  if (dtype != 0 && dtype != 1) {
    err = "dtype must be GDR_F32 or GDR_BF16";
    return false;
  }
  if (state_layout != 0 && state_layout != 1) {
    err = "state_layout must be GDR_STATE_KV or GDR_STATE_VK";
    return false;
  }
  if (static_cast<int64_t>(B) * T > INT32_MAX || static_cast<int64_t>(B) * T * H > (int64_t(1) << 40)) {
    err = "too many tokens for one call (B*T must fit in int32)";
    return false;
  }
  p.B = B;
  p.T = T;
  p.H = H;
  p.DK = DK;
  p.DV = DV;
  p.dtype = dtype;
  p.state_vk = state_layout;
  p.seqs.clear();
  if (cu == nullptr) {
    if (N != B) {
      err = "dense rows need N == B";
      return false;
    }
    for (int b = 0; b < B; ++b) p.seqs.push_back({static_cast<int64_t>(b) * T, T, 0});
  } else {
    if (B != 1) {
      err = "packed sequences (cu_seqlens) need B == 1";
      return false;
    }
    if (N < 0) {
      err = "N must be >= 0";
      return false;
    }
    if (cu[0] != 0) {
      err = "cu_seqlens[0] must be 0";
      return false;
    }
    for (int n = 0; n < N; ++n) {
      if (cu[n + 1] < cu[n]) {
        err = "cu_seqlens must be non-decreasing (entry " + std::to_string(n + 1) + ")";
        return false;
      }
      p.seqs.push_back({cu[n], static_cast<int64_t>(cu[n + 1]) - cu[n], 0});
    }
    if (static_cast<int64_t>(cu[N]) != T) {
      err = "cu_seqlens[N] must equal T";
      return false;
    }
  }
  p.N = static_cast<int>(p.seqs.size());
  int64_t c = 0;
  for (auto& s : p.seqs) {
    s.chunk_off = c;
    c += (s.len + kChunk - 1) / kChunk;
  }
  p.n_chunks = c;
  if (c > INT32_MAX / 2) {
    err = "too many chunks";
    return false;
  }
  p.pool_idx.clear();
  p.pool_size = 0;
  if (pool_idx != nullptr) {
    if (pool_size < 1) {
      err = "pool_size must be >= 1 with state_indices_host";
      return false;
    }
    std::vector<char> seen(static_cast<size_t>(pool_size), 0);
    for (int n = 0; n < p.N; ++n) {
      const int32_t i = pool_idx[n];
      if (i < 0 || i >= pool_size) {
        err = "state index " + std::to_string(i) + " of sequence " + std::to_string(n) + " is outside the pool";
        return false;
      }
      if (seen[i]) {
        err = "state index " + std::to_string(i) + " appears twice";
        return false;
      }
      seen[i] = 1;
      p.pool_idx.push_back(i);
    }
    p.pool_size = pool_size;
  }
  return true;
}

// Built tiles (must match the instantiations in scan.hip and scan2.hip).  DK =
// 256 (bfloat16) runs the generic kernel of scan.hip with its four tiles.
static bool tile_built(int dtype, int dk, int bv, int waves, int stages) {
  if (dtype == 1 && dk == 256) {
    static const int g_tiles[][3] = {{32, 2, 1}, {32, 2, 2}, {64, 4, 1}, {64, 4, 2}};
    for (auto& t : g_tiles)
      if (t[0] == bv && t[1] == waves && t[2] == stages) return true;
    return false;
  }
  if (dtype == 1 && bv == 256 && waves == 8 && stages == 2) return true;  // balanced summaries only
  static const int bf16_tiles[][3] = {{32, 2, 2}, {32, 2, 3}, {64, 2, 3}, {64, 4, 2},
                                      {64, 4, 3}, {128, 4, 2}, {128, 4, 3}};
  static const int f32_tiles[][3] = {{32, 2, 1}, {32, 2, 2}, {64, 4, 1}, {64, 4, 2}};
  if (dtype == 1) {
    for (auto& t : bf16_tiles)
      if (t[0] == bv && t[1] == waves && t[2] == stages) return true;
  } else {
    for (auto& t : f32_tiles)
      if (t[0] == bv && t[1] == waves && t[2] == stages) return true;
  }
  return false;
}

bool choose_tile(const Problem& p, const int32_t* req, int mode, int64_t rows, Tile& t, std::string& err) {
  int r[3] = {0, 0, 0};
  if (req != nullptr) {
    r[0] = req[0];
    r[1] = req[1];
    r[2] = req[2];
  } else if (const char* env = getenv("GDR_FORCE_TILE")) {
    if (sscanf(env, "%d,%d,%d", &r[0], &r[1], &r[2]) != 3) {
      err = "GDR_FORCE_TILE must be 'bv,waves,stages'";
      return false;
    }
  } else {
    // Fixed shape-class table, from measured sweeps on MI355X (bfloat16,
    // dk = dv = 128): with enough (row, head) pairs to give every CU at least
    // a quarter of a 64-column unit, 64-column blocks of 4 waves with one LDS
    // buffer (several workgroups per CU) win; with very few pairs (one long
    // sequence, a handful of heads) 32-column blocks of 2 waves give more
    // units and a shorter chain per chunk.  The summary pass reads no U for
    // its transition columns and stores no per-chunk state, so once 128-column
    // blocks alone fill the 256 CUs, the wider block (K and W read by half as
    // many workgroups) wins there (16 segments x 8 heads: 144 us against
    // 174 us for 64-column blocks), and once one 8-wave block of all 256
    // columns per (segment, head) fills them, that block (two waves per SIMD,
    // K and W staged once per segment-head) wins again (32 segments x 8
    // heads: 108 us against 128 us).  In the plain pass, once 64-column
    // blocks would exceed two per CU (the dense form, three sharing a CU) on
    // long rows (16 chunks or more per row on average), 128-column blocks
    // win: their serial chains share a CU with fewer others (8 rows of 1.3K
    // to 3.6K tokens x 48 heads: 295 us against 323 us; at 32 heads, 512
    // blocks of 64 columns, 218 us against 243 us; 24 short rows x 48 heads:
    // 95 us against 105 us).
    const int64_t pairs = rows * p.H;
    const int64_t units64 = pairs * ((mode == 1 ? p.DV + p.DK : p.DV) / 64);
    const bool long_rows = rows > 0 && p.n_chunks >= 16 * static_cast<int64_t>(p.N);
    if (p.dtype == 1) {
      r[0] = 64;
      r[1] = 4;
      r[2] = 2;
      if (mode == 0 && p.DV % 128 == 0 && units64 > 512 && long_rows) {
        r[0] = 128;
        r[1] = 4;
        r[2] = 2;
      } else if (units64 < 64) {
        r[0] = 32;
        r[1] = 2;
        r[2] = 2;
      } else if (mode == 1 && p.DK == 128 && p.DV == 128 && summary_kernel_mode(p) == 2 && pairs >= 256) {
        r[0] = 256;
        r[1] = 8;
        r[2] = 2;
      } else if (mode == 1 && p.DV % 128 == 0 && p.DK % 128 == 0 && units64 / 2 >= 256) {
        r[0] = 128;
        r[1] = 4;
        r[2] = 3;
      }
    } else {
      r[0] = 64;
      r[1] = 4;
      r[2] = 2;
      if (units64 < 512) {
        r[0] = 32;
        r[1] = 2;
        r[2] = 2;
      }
    }
  }
  const int kmode = (mode == 1) ? summary_kernel_mode(p) : 0;
  if (!tile_built(p.dtype, p.DK, r[0], r[1], r[2])) {
    err = "tile (bv=" + std::to_string(r[0]) + ", waves=" + std::to_string(r[1]) +
          ", stages=" + std::to_string(r[2]) + ") is not built for this dtype";
    return false;
  }
  if (kmode == 2) {  // blocks of bv/2 state and bv/2 transition columns
    if (r[0] / 2 > p.DV || p.DV % (r[0] / 2) != 0) {
      err = "bv/2 must divide DV for segment summaries";
      return false;
    }
  } else if (r[0] > p.DV || p.DV % r[0] != 0) {
    err = "bv must divide DV";
    return false;
  }
  if (kmode == 1 && p.DK % r[0] != 0) {
    err = "bv must divide DK for segment summaries";
    return false;
  }
  t.bv = r[0];
  t.waves = r[1];
  t.stages = r[2];
  return true;
}

int summary_kernel_mode(const Problem& p) { return (p.dtype == 1 && p.DK == p.DV) ? 2 : 1; }

int summary_split(const Problem& p, int P) {
  if (summary_kernel_mode(p) != 2 || p.DK != 128 || p.DV != 128) return 1;
  const int64_t blocks = static_cast<int64_t>(p.N) * P * p.H * 2;  // 128-column blocks of a direct pass
  return (blocks > 0 && blocks < 512) ? 2 : 1;
}

int auto_segments(const Problem& p) {
  if (!p.pool_idx.empty() || p.DK > 128 || p.DV > 128) return 0;
  int64_t chains = 0, nt_max = 0;
  for (const Seq& s : p.seqs) {
    if (s.len == 0) continue;
    chains += p.H;
    nt_max = std::max<int64_t>(nt_max, (s.len + kChunk - 1) / kChunk);
  }
  if (chains == 0 || chains * (p.DV / 64) >= 128 || nt_max < 8) return 0;
  int P = (chains <= 4 && nt_max >= 1024) ? 32 : 16;
  while (P > 1 && nt_max / P < 4) P /= 2;
  return P >= 2 ? P : 0;
}

int scan_blocks(const Problem& p, const Tile& t, int mode) {
  if (mode != 1) return p.DV / t.bv;
  return summary_kernel_mode(p) == 2 ? 2 * p.DV / t.bv : (p.DV + p.DK) / t.bv;
}

void segment_bounds(int64_t len, int P, std::vector<int64_t>& t0, std::vector<int64_t>& t1) {
  // NT chunks dealt out evenly; the first NT mod P segments get one more.
  const int64_t nt = (len + kChunk - 1) / kChunk;
  const int64_t base = nt / P, extra = nt % P;
  t0.clear();
  t1.clear();
  int64_t c = 0;
  for (int s = 0; s < P; ++s) {
    const int64_t nc = base + (s < extra ? 1 : 0);
    t0.push_back(std::min(c * kChunk, len));
    t1.push_back(std::min((c + nc) * kChunk, len));
    c += nc;
  }
}

static void finish_scan_launch(Launch& l, int H, int nblk) {
  const int64_t pairs = static_cast<int64_t>(l.rows.size()) * H;
  l.grid = static_cast<int>(8 * nblk * ((pairs + 7) / 8));
}

std::vector<Launch> plan_scan(const Problem& p, const Tile& t, int mode, int P, bool has_h0, bool has_hT,
                              int split) {
  std::vector<Row> rows;
  if (mode == 0) {
    for (int n = 0; n < p.N; ++n) {
      const Seq& s = p.seqs[n];
      const int32_t st = p.pool_idx.empty() ? n : p.pool_idx[n];  // state row (pool index if any)
      rows.push_back(Row{static_cast<int32_t>(s.bos), static_cast<int32_t>(s.len),
                         static_cast<int32_t>(s.chunk_off), has_h0 ? st : -1, has_hT ? st : -1});
    }
  } else {
    std::vector<int64_t> t0, t1;
    for (int n = 0; n < p.N; ++n) {
      const Seq& s = p.seqs[n];
      segment_bounds(s.len, P, t0, t1);
      for (int k = 0; k < P; ++k) {
        const int seg = n * P + k;
        if (mode == 1 && split == 2) {
          // halves: the first ceil(chunks / 2) chunks, then the rest
          const int64_t nc = (t1[k] - t0[k] + kChunk - 1) / kChunk;
          const int64_t mid = std::min(t0[k] + ((nc + 1) / 2) * kChunk, t1[k]);
          const int64_t lo[2] = {t0[k], mid}, hi[2] = {mid, t1[k]};
          for (int hf = 0; hf < 2; ++hf) {
            Row r;
            r.bos = static_cast<int32_t>(s.bos + lo[hf]);
            r.len = static_cast<int32_t>(hi[hf] - lo[hf]);
            r.chunk_off = static_cast<int32_t>(s.chunk_off + lo[hf] / kChunk);
            r.in_idx = -1;
            r.out_idx = 2 * seg + hf;
            rows.push_back(r);
          }
          continue;
        }
        Row r;
        r.bos = static_cast<int32_t>(s.bos + t0[k]);
        r.len = static_cast<int32_t>(t1[k] - t0[k]);
        r.chunk_off = static_cast<int32_t>(s.chunk_off + t0[k] / kChunk);
        if (mode == 1) {
          r.in_idx = -1;
          r.out_idx = seg;
        } else {
          r.in_idx = seg;
          r.out_idx = (k == P - 1 && has_hT) ? n : -1;
        }
        rows.push_back(r);
      }
    }
  }
  // longest first (stable, so equal lengths keep their order)
  std::stable_sort(rows.begin(), rows.end(), [](const Row& a, const Row& b) { return a.len > b.len; });
  const int nblk = scan_blocks(p, t, mode);
  std::vector<Launch> out;
  for (size_t i = 0; i < rows.size(); i += kMaxRows) {
    Launch l;
    l.rows.assign(rows.begin() + i, rows.begin() + std::min(rows.size(), i + kMaxRows));
    finish_scan_launch(l, p.H, nblk);
    out.push_back(std::move(l));
  }
  return out;
}

std::vector<Launch> plan_chunks(const Problem& p, int blocks_per_chunk) {
  std::vector<Launch> out;
  Launch cur;
  int64_t base = -1;
  auto flush = [&]() {
    if (!cur.rows.empty()) {
      cur.grid = cur.n_chunks * p.H * blocks_per_chunk;
      out.push_back(std::move(cur));
    }
    cur = Launch();
    base = -1;
  };
  const int64_t max_chunks = (int64_t(1) << 30) / (static_cast<int64_t>(p.H) * blocks_per_chunk);
  for (const Seq& s : p.seqs) {
    const int64_t nc = (s.len + kChunk - 1) / kChunk;
    if (nc == 0) continue;
    if (!cur.rows.empty() && (cur.rows.size() >= static_cast<size_t>(kMaxRows) || cur.n_chunks + nc > max_chunks))
      flush();
    if (base < 0) {
      base = s.chunk_off;
      cur.chunk_base = static_cast<int>(base);
    }
    cur.rows.push_back(Row{static_cast<int32_t>(s.bos), static_cast<int32_t>(s.len),
                           static_cast<int32_t>(s.chunk_off - base), -1, -1});
    cur.n_chunks += static_cast<int>(nc);
  }
  flush();
  return out;
}

}  // namespace gdr
