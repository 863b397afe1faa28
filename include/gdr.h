/*
 * gdr.h — C ABI of the chunkwise gated-delta state scan for AMD Instinct
 * MI355X (gfx950), and of its ABC diagonal-affine sibling.
 *
 * Sources of the operations (the pages the library is built from):
 *   [kev#259]  kev pull request #259 (autotune cache split by sequence count
 *              for fla's DeltaNet state-scan kernel) — the per-chunk state
 *              scan run inside each DeltaNet layer, its value-block width BV,
 *              packed variable-length batches counted from cu_seqlens, and the
 *              property that all tile configs give bit-identical output
 *              (opening section; "Why 4 sequences").
 *   [cuLA#127] cuLA pull request #127 — intracard context parallelism: a
 *              pre-scan that forms a segment's local state and its affine
 *              transition kept canonically in FP32, composed segment after
 *              segment ("Summary"; "Root cause and implementation"), and
 *              initial/final-state and transposed-state layouts ("Validation").
 *   [fla#23]   flash-linear-attention fork issue #23, "[Perf][B300]
 *              Parallelize ABC chunk state construction with affine
 *              summaries" — the ABC slot states advanced per 64-token chunk
 *              as state_out = state_in * r + c, with r from the cumulative
 *              normaliser z ("Problem"; "Proposed Dataflow").
 *
 * The recurrence (one sequence, one head; a_t = exp(g_t), b_t = beta_t):
 *     S_t = a_t (I - b_t k_t k_t^T) S_{t-1} + b_t k_t v_t^T,   o_t = scale * S_t^T q_t
 * computed per 64-token chunk in the WY form: prepare (g_cum, w, u), scan
 * (v_new = u - w S; emit S before the chunk; S <- e^{g_last} S +
 * K^T (v_new * e^{g_last - g})), output (o from q, k, v_new, h).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers without a _host suffix are DEVICE pointers owned by the caller;
 *    the library never allocates, frees or retains them.  Every device
 *    pointer must be 16-byte aligned.
 *  - `stream` is a hipStream_t (NULL = the default stream).  All work is
 *    enqueued on it, nothing is synchronised, and GDR_OK means "enqueued".
 *  - Arguments are validated completely before any launch: on an error
 *    return nothing has been enqueued and no output was written.
 *    gdr_last_error() gives a message for the calling thread.
 *  - No C++ exception crosses the ABI; the library holds no mutable global
 *    state (apart from the per-device address of the static scratch of
 *    gdr_segment_summaries_noalloc, looked up once under a lock), so
 *    concurrent calls from several threads are safe (that entry point's
 *    calls on one GPU excepted: they share its scratch).
 *  - Layouts are contiguous, time-major ("public layout", [fla#23] fixture
 *    contract):
 *        q, k, w            [B, T, H, DK]   storage dtype
 *        v, u, v_new, o     [B, T, H, DV]   storage dtype
 *        g, beta, g_cum     [B, T, H]       float32
 *        h                  [NT, H, DV, DK] storage dtype; h[c, :, j, i] = S_c[i, j]
 *                           (value-major: the state before chunk c, transposed)
 *        h0, hT             [N, H, DK, DV] float32 (GDR_STATE_KV) or
 *                           [N, H, DV, DK] float32 (GDR_STATE_VK)
 *    A packed batch uses B = 1, T = total tokens and cu_seqlens_host with N+1
 *    entries; sequence n is tokens [cu[n], cu[n+1]).  Chunks restart at each
 *    sequence start; NT = sum_n ceil(L_n / 64), sequences in order.
 *  - Supported: DK, DV in {64, 128}, float32 or bfloat16 storage, for every
 *    entry point.  With bfloat16 storage DK and DV may also be 256 (each of
 *    them; (256, 256), (256, 128), (128, 256)) for gdr_chunk_prepare,
 *    gdr_state_scan and gdr_chunk_output; the segment summaries and
 *    composition, the reverse pass and the per-channel decay entry points
 *    return GDR_ERR_UNSUPPORTED there.  Chunk size is 64 tokens.
 */
#ifndef GDR_H_
#define GDR_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GDR_OK = 0,
  GDR_ERR_INVALID_ARG = 1, /* bad pointer, size, layout or cu_seqlens        */
  GDR_ERR_UNSUPPORTED = 2, /* valid request this build has no kernel for     */
  GDR_ERR_HIP = 3          /* a HIP runtime call or launch failed            */
} gdr_status;

typedef enum { GDR_F32 = 0, GDR_BF16 = 1 } gdr_dtype;

/* Layout of h0/hT: KV = [.., DK, DV] (the state as written), VK = its transpose
 * ([cuLA#127] "Validation" lists both layouts). */
typedef enum { GDR_STATE_KV = 0, GDR_STATE_VK = 1 } gdr_state_layout;

typedef struct {
  int32_t B;                       /* batch rows; 1 for a packed batch            */
  int64_t T;                       /* tokens per row, or total packed tokens      */
  int32_t H, DK, DV;               /* heads, key width, value width               */
  int32_t N;                       /* sequences: B (dense) or len(cu_seqlens) - 1 */
  const int32_t* cu_seqlens_host;  /* N+1 host ints, or NULL for dense rows; read
                                      during the call only                        */
  gdr_dtype dtype;                 /* storage of q, k, v, w, u, v_new, o and h    */
  gdr_state_layout state_layout;   /* layout of h0 and hT                         */
  /* Indexed states ([kev#259] "Not covered": question rows whose cached states
   * are addressed by index).  NULL, or N host ints read during the call only:
   * h0 and hT are then pools of pool_size states, sequence n starts from
   * h0[idx[n]] and its final state goes to hT[idx[n]]; h0 == hT updates the
   * pool in place (each state is read by the workgroups that later overwrite
   * it, and only by them).  Indices must be distinct and in [0, pool_size);
   * other pool entries are left untouched.  Serial scan only: the segment
   * entry points and a segmented gdr_state_scan return GDR_ERR_UNSUPPORTED
   * when it is set. */
  const int32_t* state_indices_host;
  int32_t pool_size;
} gdr_problem;

/* Tile of the serial scans.  bv: value columns per workgroup (the BV of
 * [kev#259]); waves: wavefronts per workgroup, each owning bv/waves columns
 * (a multiple of 16); stages: chunks in flight per workgroup (1 = load a chunk
 * then compute it, 2 = fetch the next chunk while computing the current one,
 * 3 = two chunks ahead with two LDS buffers).  Built tiles: bfloat16 (32,2,2)
 * (32,2,3) (64,2,3) (64,4,2) (64,4,3) (128,4,2) (128,4,3); float32 (32,2,1)
 * (32,2,2) (64,4,1) (64,4,2).
 * Every supported tile gives bit-identical results.  NULL = the scheduler's
 * choice. */
typedef struct {
  int32_t bv, waves, stages;
} gdr_tile;

/* Segment-parallel final pass (see gdr_state_scan): each sequence is split
 * into n_segments chunk-aligned segments and segment s of sequence n starts
 * from seg_init[n * n_segments + s]. */
typedef struct {
  int32_t n_segments;
  const float* seg_init;           /* [N * n_segments, H, DV, DK] float32 */
} gdr_segments;

/* Number of chunks NT = sum_n ceil(L_n / 64) (rows of h); -1 on invalid input. */
int64_t gdr_num_chunks(const gdr_problem* p);

/* Chunk preparation (WY factors).  Per (sequence, head, chunk) with n valid
 * tokens, gamma = inclusive cumulative sum of g inside the chunk,
 *   A[t,i] = beta_t exp(gamma_t - gamma_i) (k_t . k_i) for i < t,
 *   T = (I + A)^-1 (forward substitution, FP32),
 *   w = T diag(beta exp(gamma)) K,   u = T diag(beta) V.
 * Writes g_cum = gamma (float32), w and u (storage dtype) for every valid
 * token; nothing past a sequence's last token.  [kev#259] opening section
 * (the scan consumes these factors). */
gdr_status gdr_chunk_prepare(const gdr_problem* p, const void* k, const void* v,
                             const float* g, const float* beta, float* g_cum, void* w,
                             void* u, void* stream);

/* The inter-chunk state scan ([kev#259] opening section): for every
 * (sequence, head), serially over its chunks c with n valid tokens,
 *   h[c] = S;  v_new = u_c - w_c S;  S <- e^{g_last} S + K_c^T (v_new * e^{g_last - g}),
 * g_last = g_cum of the chunk's last valid token; rows past n are masked.
 * S starts from h0[n] (NULL = zeros) and hT[n] receives the final state.
 * h (NULL = not written) and v_new (NULL = not written) use the storage
 * dtype; S is held in FP32 throughout.
 * With `seg` non-NULL this is the segmented final pass of [cuLA#127]: every
 * segment runs from seg->seg_init (h0 is then ignored), so segments of one
 * sequence run in parallel; hT is written by each sequence's last segment.
 * Results are bit-identical for every tile and between dense rows and the
 * same rows packed with cu_seqlens. */
gdr_status gdr_state_scan(const gdr_problem* p, const gdr_tile* tile, const gdr_segments* seg,
                          const void* k, const void* w, const void* u, const float* g_cum,
                          const float* h0, void* h, void* v_new, float* hT, void* stream);

/* Chunk output: for token t of chunk c (same sequence),
 *   o_t = scale * ( e^{gamma_t} q_t^T S_c + sum_{i <= t in chunk} e^{gamma_t - gamma_i} (q_t . k_i) v_new_i ),
 * S_c read from h (storage dtype, value-major).  Equals scale * S_t^T q_t of the
 * token recurrence.  Writes o for every valid token. */
gdr_status gdr_chunk_output(const gdr_problem* p, const void* q, const void* k,
                            const void* v_new, const void* h, const float* g_cum, float scale,
                            void* o, void* stream);

/* The state scan with the chunk output fused into it: the h, v_new and hT of
 * gdr_state_scan and the o of gdr_chunk_output on them, bit for bit, from one
 * pass over the chunks (the two definitions above: [kev#259] opening section
 * for the scan; the output formula of gdr_chunk_output).  The pre-chunk state
 * and v_new of every chunk feed the output on chip, so they are not read
 * back from memory.  Fused for bfloat16, DK 64 or 128, DV <= 128 and the
 * tiles (bv 64 or 128, 4 waves, 2 stages); with tile NULL the planner's tile
 * when it is one of those, else (64, 4, 2).  There h and v_new may be NULL
 * (not written).  Any other problem or explicit tile runs gdr_state_scan and
 * then gdr_chunk_output, and then h and v_new must be given (else
 * GDR_ERR_UNSUPPORTED).  q [B, T, H, DK] and o [B, T, H, DV] in the storage
 * dtype, layouts and the other arguments as in the two calls; seg as in
 * gdr_state_scan (the segmented final pass). */
gdr_status gdr_state_scan_output(const gdr_problem* p, const gdr_tile* tile, const gdr_segments* seg,
                                 const void* q, const void* k, const void* w, const void* u,
                                 const float* g_cum, const float* h0, float scale, void* h,
                                 void* v_new, float* hT, void* o, void* stream);

/* The whole forward step of the chunkwise form in one pass over the chunks:
 * the chunk prepare (gdr_chunk_prepare: gamma, the WY factors w and u), the
 * state scan (gdr_state_scan) and the chunk output (gdr_chunk_output), with
 * w and u formed per chunk on chip instead of going through memory.  The
 * same arithmetic as gdr_chunk_prepare followed by gdr_state_scan_output, so
 * o, h, v_new, hT and g_cum are the same bits.  bfloat16 storage, DK = 128,
 * DV a multiple of 64 (64-column blocks, four waves); any other problem
 * returns GDR_ERR_UNSUPPORTED (run the two calls).  Arguments as in those
 * calls: q, k [B, T, H, DK], v [B, T, H, DV], g, beta [B, T, H] (FP32), h0
 * (nullable), o [B, T, H, DV]; g_cum, h, v_new and hT may be NULL (not
 * written).  Plain pass only (no segments); indexed states as in
 * gdr_state_scan.  No workspace. */
gdr_status gdr_chunk_forward(const gdr_problem* p, const void* q, const void* k, const void* v,
                             const float* g, const float* beta, const float* h0, float scale,
                             float* g_cum, void* h, void* v_new, float* hT, void* o, void* stream);

/* Segment summaries, the pre-scan of [cuLA#127] ("Root cause and
 * implementation"): each sequence is split into n_segments chunk-aligned
 * segments (NT_n chunks dealt out evenly, the first NT_n mod P segments one
 * more).  For segment s the chunk recurrence runs from zero on the value
 * columns (local state S_loc) and from the identity with zero values on DK
 * extra columns (the transition M_s, the product of the segment's
 * per-token transitions), so that a state entering the segment leaves as
 * M_s S_in + S_loc.  Both are FP32:
 *   seg_state  [N * P, H, DV, DK]   S_loc, value-major
 *   seg_trans  [N * P, H, DK, DK]   M_s, row-major (M[i][j]) */
gdr_status gdr_segment_summaries(const gdr_problem* p, const gdr_tile* tile, int32_t n_segments,
                                 const void* k, const void* w, const void* u,
                                 const float* g_cum, float* seg_state, float* seg_trans,
                                 void* stream);

/* Device workspace (bytes) gdr_segment_summaries_ws uses for this problem and
 * segment count; 0 when the summaries are formed directly, and also for an
 * invalid problem or n_segments < 1 (then gdr_last_error() says why; "" when
 * the problem is valid).  Host only. */
size_t gdr_segment_summaries_workspace_size(const gdr_problem* p, int32_t n_segments);

/* gdr_segment_summaries with a caller-owned device workspace (16-byte
 * aligned, at least gdr_segment_summaries_workspace_size bytes, else
 * GDR_ERR_INVALID_ARG; NULL or a zero size runs the direct form).  When the
 * size is nonzero the (segment, head) chains alone would leave most of the
 * GPU idle, so every segment is cut at half its chunk count, the two halves'
 * summaries are formed in parallel into the workspace (each from zero and
 * from the identity), and each segment's pair is composed by the same rule as
 * gdr_segment_compose ([cuLA#127] "Root cause and implementation": segments
 * are composed one after another), in FP32:
 *   S_loc = M_b S_loc(a) + S_loc(b),   M_s = M_b M_a   (a first half, b second).
 * Same outputs and layouts as gdr_segment_summaries; equal to them up to
 * rounding, and bit-identical for every tile.  The workspace holds nothing
 * after the call. */
gdr_status gdr_segment_summaries_ws(const gdr_problem* p, const gdr_tile* tile, int32_t n_segments,
                                    const void* k, const void* w, const void* u,
                                    const float* g_cum, float* seg_state, float* seg_trans,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* gdr_segment_summaries_ws for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the half-segment workspace is a static device array inside the
 * library, GDR_NOALLOC_SCRATCH_BYTES per GPU, held until the process ends.
 * The call allocates nothing.  Same arguments (less the workspace), outputs
 * and results as gdr_segment_summaries_ws given a workspace of
 * gdr_segment_summaries_workspace_size bytes; a problem that needs more than
 * GDR_NOALLOC_SCRATCH_BYTES returns GDR_ERR_INVALID_ARG before any launch
 * (64K tokens x 8 heads x 16 segments at DK = DV = 128 needs 32 MiB; with
 * 16 segments of one 64K sequence up to 12 heads fit).
 * Every call on one GPU uses that GPU's one array: calls that overlap on the
 * same GPU (other streams, other threads) race and must be serialised by the
 * caller.  The array holds nothing a later call relies on. */
#define GDR_NOALLOC_SCRATCH_BYTES ((size_t)48 << 20)
gdr_status gdr_segment_summaries_noalloc(const gdr_problem* p, const gdr_tile* tile, int32_t n_segments,
                                         const void* k, const void* w, const void* u, const float* g_cum,
                                         float* seg_state, float* seg_trans, void* stream);

/* Segment composition ([cuLA#127] "Root cause and implementation"), in FP32,
 * serially over the segments of each sequence:
 *   S_init(0) = h0[n] (NULL = zeros);  S_init(s+1) = M_s S_init(s) + S_loc(s).
 * seg_init [N * P, H, DV, DK] value-major; hT (nullable) receives
 * M_{P-1} S_init(P-1) + S_loc(P-1) in the state_layout of p. */
gdr_status gdr_segment_compose(const gdr_problem* p, int32_t n_segments, const float* seg_state,
                               const float* seg_trans, const float* h0, float* seg_init,
                               float* hT, void* stream);

/* ABC slot-state construction ([fla#23] "Problem", "Proposed Dataflow").
 * Per batch row and head, with slot logits s_t and z_t = log(e^{z_{t-1}} + e^{s_t})
 * (z_0 = -inf, no initial state), per 64-token chunk c ending at token e:
 *   r_c = exp(z_{prev chunk end} - z_e),   E_t = exp(s_t - z_e),
 *   Hk <- Hk * r_c[None, :] + K_c^T E      ([K x M], slots on columns)
 *   Hv <- Hv * r_c[:, None] + E^T V_c      ([M x V], slots on rows)
 * with the chunk contributions formed in FP32 and the states kept in FP32.
 * Layouts: k [B, T, H, K], v [B, T, H, V], s [B, T, H, M] (storage dtype);
 * z (nullable) [B, T, H, M] float32; hk [B, NC, H, K, M] and hv [B, NC, H, M, V]
 * the states before every chunk (storage dtype); hk_final [B, H, K, M] and
 * hv_final [B, H, M, V] float32 (nullable).  Supported: K, V multiples of 64,
 * M = 32 or 64 ([fla#23] "Fixture-First Correctness Contract" names both),
 * bfloat16 storage. */
typedef struct {
  int32_t B;
  int64_t T;
  int32_t H, K, M, V;
  gdr_dtype dtype;
} abc_problem;

/* Reverse (gradient) pass ([fla#23] "Problem": the reverse kernel that walks
 * the state chunk by chunk; "Proposed Dataflow", item 4: the reverse dH
 * recurrence).  For a loss L with upstream gradients dO = dL/do (storage
 * dtype, like v) and dhT = dL/dhT (float32, nullable = zero), per chunk c of
 * each sequence with gamma = the chunk-local cumulative log decay (g_cum),
 * gamma_C its last valid value and P[t][i] = (q_t . k_i) e^{gamma_t - gamma_i}
 * for i <= t (else 0):
 *   dh[c]      = dL/dS after chunk c as the input of the rest of the sequence
 *                (dhT after the last chunk)
 *   dv_local   = scale P^T dO                          (chunk-local part)
 *   dv_new     = diag(e^{gamma_C - gamma}) K dh[c] + dv_local
 *                (dL/d v_new, the gradient of the forward scan's write vectors)
 *   dh[c - 1]  = e^{gamma_C} dh[c] + scale Q^T diag(e^gamma) dO - W^T dv_new
 *   dh0        = the same expression after the first chunk (dL/dh0).
 * Bfloat16 storage only; the pool (state_indices_host) is not supported here. */

/* dv_local for every chunk, chunk-parallel: q, k [B,T,H,DK], g_cum [B,T,H],
 * dO [B,T,H,DV] -> dv_local [B,T,H,DV] (storage dtype).  Rows past a
 * sequence's last token are not written. */
gdr_status gdr_chunk_dv_local(const gdr_problem* p, const void* q, const void* k, const float* g_cum, const void* dO,
                              float scale, void* dv_local, void* stream);

/* The reverse state scan: serial over each sequence's chunks, last to first.
 * Inputs q, k, w (from gdr_chunk_prepare), g_cum, dO, dv_local (from
 * gdr_chunk_dv_local), dhT (nullable, [N,H,DK,DV] or [N,H,DV,DK] by
 * state_layout).  Outputs (each nullable): dh [NT,H,DV,DK] storage dtype,
 * value-major like h; dv_new_grad [B,T,H,DV] storage dtype; dh0 float32 in
 * the state layout. */
gdr_status gdr_state_scan_bwd(const gdr_problem* p, const void* q, const void* k, const void* w, const float* g_cum,
                              const void* dO, const void* dv_local, const float* dhT, float scale, void* dh,
                              void* dv_new_grad, float* dh0, void* stream);

/* Device workspace abc_affine_scan needs (bytes). */
size_t abc_workspace_size(const abc_problem* p);

gdr_status abc_affine_scan(const abc_problem* p, const void* k, const void* v, const void* s,
                           float* z, void* hk, void* hv, float* hk_final, float* hv_final,
                           void* workspace, size_t workspace_bytes, void* stream);

/* ABC read per 64-token chunk ([fla#23] "Problem": chunk_abc, the operator
 * whose forward reads the slot states).  After token t's update the states
 * are read as score_t = scale Hk_t^T q_t, p_t = softmax over the M slots of
 * score_t, o_t = Hv_t^T p_t; per chunk this combines the pre-chunk states
 * hk[c], hv[c] with the chunk's own tokens.  Inputs: q, k [B, T, H, K],
 * v [B, T, H, V], s [B, T, H, M] (storage dtype), z [B, T, H, M] float32 and
 * hk [B, NC, H, K, M], hv [B, NC, H, M, V] as abc_affine_scan writes them.
 * Outputs: o [B, T, H, V] (storage dtype); p_out (nullable) [B, T, H, M] the
 * slot weights.  Bfloat16 storage, M = 32 or 64, (K, V) in {(64, 128), (128, 128),
 * (128, 256), (256, 256), (256, 512)} (else GDR_ERR_UNSUPPORTED). */
gdr_status abc_chunk_output(const abc_problem* p, const void* q, const void* k, const void* v, const void* s,
                            const float* z, const void* hk, const void* hv, float scale, void* o, void* p_out,
                            void* stream);

/* ABC reverse (dH) recurrence ([fla#23] "Problem": the reverse kernel that
 * walks every state tile chunk by chunk; "Proposed Dataflow", item 4: the
 * same producer / ordered-scan split for the reverse recurrence).  The slot
 * states are read after every token as score_t = scale Hk_t^T q_t (M slot
 * scores) and o_t = Hv_t^T p_t (V outputs).  Given the gradients dscore =
 * dL/dscore and dO = dL/do (storage dtype) and of the final states (float32,
 * nullable = zero), per chunk c ending at token e
 *   dhk[c], dhv[c] = dL/d(state after chunk c) as the input of the tokens
 *                    after it (the final states' gradient for the last chunk)
 * by the reverse diagonal-affine walk, r_c = exp(zc[c-1] - zc[c]):
 *   dhk[c-1] = dhk[c] * r_c[None, :] + scale Q_c^T (dscore_c * e^{zc[c-1] - z})
 *   dhv[c-1] = r_c[:, None] * dhv[c] + (p_c * e^{zc[c-1] - z})^T dO_c
 * Layouts: q [B, T, H, K], dscore, p [B, T, H, M], dO [B, T, H, V] (storage
 * dtype); z [B, T, H, M] float32, the normaliser abc_affine_scan writes;
 * dhk_final [B, H, K, M], dhv_final [B, H, M, V] float32 (nullable); outputs
 * dhk [B, NC, H, K, M], dhv [B, NC, H, M, V] in the storage dtype.  Same
 * shape support as abc_affine_scan; all pointers 16-byte aligned. */
size_t abc_bwd_workspace_size(const abc_problem* p);

gdr_status abc_affine_scan_bwd(const abc_problem* p, const void* q, const void* dscore, const void* pw,
                               const void* dO, const float* z, const float* dhk_final, const float* dhv_final,
                               float scale, void* dhk, void* dhv, void* workspace, size_t workspace_bytes,
                               void* stream);

/* ------------------------------------------------------------------------
 * Per-key-channel decay (the FlashKDA-style gate of [cuLA#127] "Summary" and
 * "Root cause and implementation": the serial path whose pre-scan that page
 * parallelises; no recurrence is printed there).  Recurrence, one sequence and
 * one head, with a per-channel decay a_t = exp(g_t) in R^DK:
 *     S_t = (I - b_t k_t k_t^T) diag(a_t) S_{t-1} + b_t k_t v_t^T,  o_t = scale * S_t^T q_t
 * (every key row of the state decays by its own factor, then the delta-rule
 * write on the decayed state; with all channels equal it is the recurrence
 * above).  Per 64-token chunk, Gam = chunk-local inclusive cumulative sum of g
 * per channel:
 *   A[t,i] = b_t sum_d k_td k_id e^{Gam_td - Gam_id} (i < t), T = (I + A)^-1,
 *   w = T diag(b) (K * e^{Gam}),  u = T diag(b) V,
 *   kg = K * e^{Gam_last - Gam},  decay = e^{Gam_last}   (per channel)
 *   scan:   h[c] = S;  v_new = u - w S;  S <- diag(decay) S + kg^T v_new
 *   output: o_t = scale ((q_t * e^{Gam_t})^T S_c + sum_{i<=t} P[t,i] v_new_i),
 *           P[t,i] = sum_d q_td k_id e^{Gam_td - Gam_id}
 * Layouts as above, except g and g_cum [B, T, H, DK] float32, kg [B, T, H, DK]
 * (storage dtype) and decay [NT, H, DK] float32 (one vector per chunk and
 * head, chunks numbered like the rows of h).  Bfloat16 storage only.
 * Input range: the intra-chunk products are formed per 16-token block with
 * the block's first token as reference, which stays finite while every
 * channel's log decay is at least -5 per token; smaller values (a decay
 * below e^-5 in one token) can overflow to inf/NaN. */

/* Chunk preparation: writes g_cum, w, u and kg for every valid token and the
 * channel decays of every chunk. */
gdr_status kda_chunk_prepare(const gdr_problem* p, const void* k, const void* v, const float* g, const float* beta,
                             float* g_cum, void* w, void* u, void* kg, float* decay, void* stream);

/* The inter-chunk state scan with per-channel decay: gdr_state_scan's
 * contract (tiles, segmented final pass, pools, layouts, bit-identity across
 * tiles) with kg in place of k and the chunk decays in place of g_cum. */
gdr_status kda_state_scan(const gdr_problem* p, const gdr_tile* tile, const gdr_segments* seg, const void* kg,
                          const void* w, const void* u, const float* decay, const float* h0, void* h, void* v_new,
                          float* hT, void* stream);

/* Segment summaries with per-channel decay (gdr_segment_summaries' contract;
 * the transition of a chunk is diag(decay) - kg^T w).  Compose them with
 * gdr_segment_compose. */
gdr_status kda_segment_summaries(const gdr_problem* p, const gdr_tile* tile, int32_t n_segments, const void* kg,
                                 const void* w, const void* u, const float* decay, float* seg_state, float* seg_trans,
                                 void* stream);

/* Chunk output with per-channel decay (o for every valid token). */
gdr_status kda_chunk_output(const gdr_problem* p, const void* q, const void* k, const void* v_new, const void* h,
                            const float* g_cum, float scale, void* o, void* stream);

/* Human-readable name of a status code. */
const char* gdr_status_string(gdr_status s);
/* Message of the last failed call on this thread ("" if none). */
const char* gdr_last_error(void);

/* The state scan with the segmentation chosen by the scheduler ([kev#259]
 * "Why 4 sequences": one long state, or a few, leave most of the GPU idle in
 * the serial scan; [cuLA#127] "Summary": the same scan split into segments
 * whose affine summaries are composed in FP32).  gdr_plan_segments gives the
 * segment count P it takes for this problem: 0 = the serial scan (many
 * sequence-head chains, short sequences, state pools, DK or DV of 256),
 * else P >= 2.  gdr_state_scan_auto then runs, on `stream`:
 *   P = 0: gdr_state_scan_output (q and o given) or gdr_state_scan;
 *   P > 0: gdr_segment_summaries_ws, gdr_segment_compose (from h0) and the
 *          segmented final pass (with the chunk output fused when q and o
 *          are given), the summaries and initial states in the workspace.
 * Results are those of the explicit calls with n_segments = P, bit for bit.
 * workspace: device memory of at least gdr_state_scan_auto_workspace_size
 * bytes (0 when P = 0; NULL is then allowed), 16-byte aligned; it holds
 * nothing after the call.  q and o are given together or not at all; other
 * arguments as in gdr_state_scan_output.  gdr_plan_segments returns -1 for
 * an invalid problem. */
int32_t gdr_plan_segments(const gdr_problem* p);
size_t gdr_state_scan_auto_workspace_size(const gdr_problem* p);
gdr_status gdr_state_scan_auto(const gdr_problem* p, const void* q, const void* k, const void* w, const void* u,
                               const float* g_cum, const float* h0, float scale, void* h, void* v_new, float* hT,
                               void* o, void* workspace, size_t workspace_bytes, void* stream);

/* Scheduler introspection (host only, no GPU needed): the tile and grid the
 * scan would use (n_segments > 0: the summary pass as gdr_segment_summaries_ws
 * runs it with its workspace, i.e. on half segments when that form applies).
 * out[0..5] = bv, waves, stages, workgroups, launches, rows per launch (max). */
gdr_status gdr_plan_query(const gdr_problem* p, const gdr_tile* tile, int32_t n_segments,
                          int64_t out[6]);

#ifdef __cplusplus
}
#endif

#endif /* GDR_H_ */
