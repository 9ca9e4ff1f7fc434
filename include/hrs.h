/*
 * hrs.h - hybrid recurrent state: verify-span checkpoints, greedy acceptance
 * and on-device rollback for Gated DeltaNet (GDN) layers, on AMD MI355X
 * (gfx950).
 *
 * The library implements the data-parallel hot path of verifying a
 * speculative-decoding draft block through the recurrent layers of a hybrid
 * Qwen3.5/3.6-style target:
 *
 *   conv1d_verify_span  causal depthwise conv over the span, conv state
 *                       captured after every position
 *   gdn_verify_span     gated delta rule over the span (chain or draft tree),
 *                       F32 state checkpoint after every position
 *   accept_greedy       target argmax per position and the longest matching
 *                       prefix / root path
 *   rollback_restore    restore the accepted checkpoint of every layer on the
 *                       device, index read on the device, no replay
 *   ring_set_2d / ring_get_2d
 *                       batched feature-ring row copies with wraparound
 *
 * and, beside them: gdn_verify_span_from, conv1d_verify_span_nocapture and
 * conv_state_advance (zero-copy rollback), gdn_layer_verify_span (one layer
 * fused into one kernel) and gdn_span_chunked (long spans in chunks).
 *
 * Conventions shared by every entry point
 * ----------------------------------------
 *  - Memory: every device buffer is allocated and owned by the caller. The
 *    library allocates and frees nothing and keeps no pointer after a call
 *    returns. Host arrays (parent, runs) are read during the call only.
 *  - Streams: every device call is asynchronous on `stream` (a hipStream_t
 *    passed as void*; NULL means the null stream). Nothing synchronises.
 *  - Layout: dense, row-major, dims as written. Multi-layer buffers carry a
 *    leading [L] dim; per-layer calls take pointers into one layer.
 *  - Alignment: device pointers must be 16-byte aligned.
 *  - Errors: a negative return means nothing was launched (fail closed),
 *    except HRS_EDEVICE, which reports that the launch itself failed.
 *    Every argument check runs on the host before any HIP call, so the
 *    checks also work on a machine without a GPU.
 *  - Thread safety: the library holds no mutable global state shared
 *    between threads; each thread keeps a record of its last HIP error (see
 *    hrs_last_hip_error) and a cache of the device attributes its launches
 *    need (compute units, LDS per block), keyed by the current device.
 *  - Determinism: results are bit-identical from run to run, and the
 *    arithmetic of one position does not depend on the span length or on the
 *    tree topology.
 *
 * Sources (the pages this path comes from):
 *  [P1] lucebox PR #533, "feat: DFlash support for tensor-parallel Qwen3.6
 *       targets": Changes, Verification, Sustained performance.
 *  [P2] openinfer PR #626, "feat(qwen35): add opt-in DFlash speculative
 *       decoding": Summary, What Changed, Future Work.
 *  [P3] lucebox PR #506, "perf(dflash): split-chain fast rollback with F32
 *       SSM checkpoints (+29% decode)": Summary, Memory trade-off, Safety
 *       boundary, Verification.
 *  [GDN] Yang, Kautz, Hatamizadeh, "Gated Delta Networks: Improving Mamba2
 *       with Delta Rule", ICLR 2025: the gated delta rule.
 */
#ifndef HRS_H
#define HRS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HRS_ABI_VERSION 1

/* Largest span (root + drafts) a call accepts. */
#define HRS_MAX_POS 64

typedef enum {
  HRS_OK = 0,
  HRS_EINVAL = -1,       /* bad size, NULL pointer or dtype combination  */
  HRS_EGEOMETRY = -2,    /* draft geometry rejected by the guard          */
  HRS_EALIGN = -3,       /* device pointer not 16-byte aligned            */
  HRS_EDEVICE = -4,      /* the HIP launch failed                         */
  HRS_EUNSUPPORTED = -5  /* valid request outside the built kernel set    */
} hrs_status;

typedef enum { HRS_F32 = 0, HRS_BF16 = 1 } hrs_dtype;

typedef enum { HRS_CHAIN = 0, HRS_TREE = 1 } hrs_topology;

/* Verdicts of the geometry guard (see hrs_validate_tree). */
typedef enum {
  HRS_GEOM_OK = 0,
  HRS_GEOM_NULL = 1,       /* no parent array where one is required        */
  HRS_GEOM_TRUNCATED = 2,  /* n_pos outside [1, HRS_MAX_POS]               */
  HRS_GEOM_ROOT = 3,       /* parent[0] != -1, or a second root            */
  HRS_GEOM_RANGE = 4,      /* parent[i] < -1 or parent[i] >= n_pos         */
  HRS_GEOM_FORWARD = 5,    /* i <= parent[i] (self, cyclic, forward)       */
  HRS_GEOM_NOT_CHAIN = 6   /* chain required but parent[i] != i - 1        */
} hrs_geometry_class;

/*
 * hrs_validate_tree - the fail-closed geometry guard ([P3] Safety boundary:
 * sibling, malformed-root, skipped-parent, cyclic/forward-parent,
 * out-of-range, truncated and null geometry are rejected before execution).
 *
 * parent: host array of n_pos entries; position 0 is the committed root
 *         (parent -1) and every other position names an earlier position.
 * require_chain: nonzero = only the root-inclusive pure chain
 *         (parent[i] == i - 1) is accepted, as on [P3]; zero = any tree in
 *         topological order (draft trees, [P1] Verification: DDTree).
 * geometry_class: optional out (may be NULL), one hrs_geometry_class; the
 *         lowest-index offending position decides.
 * Returns HRS_OK or HRS_EGEOMETRY. Host only; touches no device.
 */
int hrs_validate_tree(const int32_t* parent, int32_t n_pos, int32_t require_chain,
                      int32_t* geometry_class);

/* ------------------------------------------------------------------------ */
/* GDN verify span                                                          */
/* ------------------------------------------------------------------------ */

typedef struct {
  int32_t n_req;      /* R  requests in the batch                          */
  int32_t n_pos;      /* T  span positions: committed root + K drafts      */
  int32_t n_kheads;   /* Hk key heads                                      */
  int32_t n_vheads;   /* Hv value heads; Hv % Hk == 0                      */
  int32_t d_k;        /* key dim: 64 or 128                                */
  int32_t d_v;        /* value dim: multiple of 16, at most 256            */
  hrs_dtype in_dtype; /* dtype of q, k, v, a, b                            */
  float q_scale;      /* q is multiplied by this after widening (1.0 = none) */
  hrs_topology topo;  /* HRS_CHAIN or HRS_TREE                             */
  const int32_t* parent; /* host [n_req][n_pos] when topo == HRS_TREE, else
                            ignored (may be NULL)                          */
} hrs_gdn_desc;

/*
 * gdn_verify_span - the gated delta rule ([GDN]) over a verify span, with an
 * F32 state checkpoint after every position ([P3] Summary: F32 SSM
 * checkpoints captured during verify for rollback without replay; [P3]
 * Verification: the GDN op writes every intermediate state to a persist
 * buffer).
 *
 * Per request r, value head h (key head g = h / (Hv/Hk)), position t whose
 * parent is p (chain: p = t - 1), with P = state[r][h] when p == -1 else
 * ckpt[r][p][h]:
 *     u        = P k_t[g]
 *     S_t      = a_t[h] P + b_t[h] (v_t[h] - a_t[h] u) k_t[g]^T
 *                (= a P (I - b k k^T) + b v k^T)
 *     ckpt[r][t][h] = S_t            (float32)
 *     out[r][t][h]  = S_t (q_scale q_t[g])
 * S is d_v rows (value dims) by d_k columns (key dims). The math is float32
 * with bf16 inputs widened exactly.
 *
 * Layouts:  q, k  [R][T][Hk][d_k]      in_dtype
 *           v     [R][T][Hv][d_v]      in_dtype
 *           a, b  [R][T][Hv]           in_dtype (decay and write strength)
 *           state [R][Hv][d_v][d_k]    float32
 *           ckpt  [R][T][Hv][d_v][d_k] float32
 *           out   [R][T][Hv][d_v]      float32
 * ckpt != NULL: state is read only; every position is captured.
 * ckpt == NULL: no capture ([P3] review: rollback storage only when
 *           explicitly requested); chain only; the state after the last
 *           position is written back to `state` (plain decode when T == 1).
 * Tree geometry is checked with hrs_validate_tree(require_chain = 0) for
 * every request before anything is launched. Errors: HRS_EINVAL,
 * HRS_EALIGN, HRS_EGEOMETRY, HRS_EUNSUPPORTED (d_k/d_v outside the built
 * set), HRS_EDEVICE.
 */
int gdn_verify_span(const hrs_gdn_desc* desc, const void* q, const void* k,
                    const void* v, const void* a, const void* b, float* state,
                    float* ckpt, float* out, void* stream);

/* Where a span's initial state comes from when it is not `state`. */
typedef struct {
  const float* ckpt;    /* device: the previous span's checkpoints of this layer,
                           [R][n_pos][Hv][d_v][d_k] float32 */
  const int32_t* node;  /* device [R]: the accepted position of that span
                           (accept_node of accept_greedy) */
  int32_t n_pos;        /* positions of the previous span, in [1, HRS_MAX_POS] */
} hrs_span_source;

/*
 * gdn_verify_span_from - zero-copy rollback: gdn_verify_span whose initial
 * state for request r is src->ckpt[r][src->node[r]], read in place on the
 * device, instead of `state`. Rolling back to the accepted checkpoint then
 * costs nothing: no copy into `state` happens at all ([P3] Summary restores
 * the accepted F32 checkpoint; this reads it where it already is). Capture is
 * required (ckpt != NULL) and ckpt must not overlap src->ckpt, so callers
 * alternate two checkpoint buffers between consecutive spans. A request whose
 * node is outside [0, src->n_pos) writes no checkpoint or output; status
 * (optional device int32, may be NULL) receives the number of such requests.
 * The canonical state can be materialised any time with rollback_restore.
 * Arithmetic, layouts and other errors as gdn_verify_span.
 */
int gdn_verify_span_from(const hrs_gdn_desc* desc, const hrs_span_source* src, const void* q,
                         const void* k, const void* v, const void* a, const void* b, float* ckpt,
                         float* out, int32_t* status, void* stream);

/*
 * gdn_verify_span_timed - gdn_verify_span whose kernel dispatch also records
 * two caller-created hipEvent_t (from the same HIP runtime as `stream`):
 * `start_event` as the kernel starts and `stop_event` as it ends. The events
 * travel inside the dispatch, so no extra command sits between kernels and
 * the interval is the kernel's own execution. Either event may be NULL.
 * Measurement support; arguments, results and errors as gdn_verify_span.
 */
int gdn_verify_span_timed(const hrs_gdn_desc* desc, const void* q, const void* k,
                          const void* v, const void* a, const void* b, float* state,
                          float* ckpt, float* out, void* stream, void* start_event,
                          void* stop_event);

/* Longest span gdn_span_chunked accepts. */
#define HRS_MAX_CHUNKED_POS (1 << 20)

typedef struct {
  hrs_gdn_desc gdn;     /* shapes, input dtype, q_scale; topo must be HRS_CHAIN */
  int32_t log_gates;    /* nonzero: `a` holds log decays g_t = log a_t (<= 0),
                           so a_t = exp(g_t); zero: `a` holds a_t itself */
  hrs_dtype out_dtype;  /* dtype of `out`: HRS_F32, or HRS_BF16 (each output
                           rounded to the nearest bf16, ties to even) */
} hrs_chunked_desc;

/* Bytes of device workspace gdn_span_chunked needs for this descriptor:
 * n_req x n_vheads x min(ceil(n_pos / 64), 32) x 20,992 (one record of T,
 * P T and the decays per request, value head and chunk of a 32-chunk
 * segment; 21.5 MB for one request of 32 heads at any length from 2,048
 * positions). 0 for a NULL descriptor or sizes out of range. */
size_t gdn_span_chunked_workspace_bytes(const hrs_chunked_desc* desc);

/*
 * gdn_span_chunked - the gated delta rule of gdn_verify_span over a long
 * chain span (prefill length, up to HRS_MAX_CHUNKED_POS positions), computed
 * by chunks of 64 positions in the chunkwise form of the delta rule ([GDN]:
 * the hardware-efficient chunkwise algorithm with the WY/UT representation).
 * Inside a chunk starting from state S_0 the written values
 *     w_t = b_t (v_t - a_t S_{t-1} k_t)
 * solve the unit lower-triangular system
 *     w_t + sum_{j<t} b_t G[t][j] (k_t . k_j) w_j = b_t (v_t - g_t S_0 k_t),
 * G[t][j] = a_{j+1}...a_t, g_t = a_0...a_t (products inside the chunk, so
 * zero or tiny decays are exact), i.e. W = T Y with T the inverse of the
 * system's matrix; then S_t = a_t S_{t-1} + w_t k_t^T and o_t = S_t
 * (q_scale q_t) as in gdn_verify_span. Same mathematics, different rounding
 * order: results agree with gdn_verify_span to f32 rounding, not bit for bit.
 *
 * Arguments, layouts and capture as gdn_verify_span, chain only
 * (desc->gdn.topo must be HRS_CHAIN; parent is ignored), with two variants:
 * log-space gates and bf16 outputs (`out` [R][T][Hv][d_v] in out_dtype).
 * ckpt != NULL writes every position's state and leaves `state` unchanged;
 * ckpt == NULL updates `state` in place to the state after the last
 * position. workspace: caller-owned device memory of at least
 * gdn_span_chunked_workspace_bytes(desc) bytes, 16-byte aligned, contents
 * ignored and overwritten (the per-chunk T, P T and decays; spans longer
 * than 32 chunks reuse it segment by segment, two launches per segment).
 * Errors: HRS_EINVAL (sizes, NULL pointers or workspace, a workspace smaller
 * than required, n_pos outside [1, HRS_MAX_CHUNKED_POS], out_dtype),
 * HRS_EALIGN, HRS_EUNSUPPORTED (tree topology; d_k or d_v other than 128),
 * HRS_EDEVICE.
 */
int gdn_span_chunked(const hrs_chunked_desc* desc, const void* q, const void* k, const void* v,
                     const void* a, const void* b, float* state, float* ckpt, void* out,
                     void* workspace, size_t workspace_bytes, void* stream);

typedef struct {
  hrs_gdn_desc gdn;    /* shapes, dtype, q_scale and topology of the span */
  int32_t conv_width;  /* W of the conv; 4 is built                        */
  int32_t silu;        /* nonzero: SiLU after the conv (the layer's order)  */
  float l2_eps;        /* added to |q|^2 and |k|^2 before the square root   */
} hrs_gdn_layer_desc;

/*
 * gdn_layer_verify_span - one GDN layer's verify span in the layer's own
 * order, in one kernel: the causal depthwise conv of the projected channels
 * (as conv1d_verify_span, optional SiLU), split into q, k and v heads, q and
 * k scaled to unit L2 norm per head, then the gated delta rule with a
 * checkpoint after every position (as gdn_verify_span). The conv and
 * recurrent states are the layer's hybrid state ([P2] What Changed); the
 * recurrence and checkpoints are those of gdn_verify_span ([GDN]; [P3]
 * Summary). The conv output never leaves the chip.
 *
 * Per request r and position t with conv output y_t (float32, C channels,
 * C = 2 Hk d_k + Hv d_v, channel order [q heads | k heads | v heads]):
 *     q_t[g] = y_t[g d_k .. ) / sqrt(|.|^2 + l2_eps)
 *     k_t[g] = y_t[Hk d_k + g d_k .. ) / sqrt(|.|^2 + l2_eps)
 *     v_t[h] = y_t[2 Hk d_k + h d_v .. )
 * then ckpt and out exactly as gdn_verify_span with q_scale applied to the
 * normalised q.
 *
 * Layouts:  x          [R][T][C]        gdn.in_dtype
 *           conv_w     [C][W]           gdn.in_dtype; w[c][W-1] multiplies x_t
 *           conv_state [R][W-1][C]      gdn.in_dtype, read only
 *           a, b       [R][T][Hv]       gdn.in_dtype
 *           state      [R][Hv][d_v][d_k] float32, read only
 *           ckpt, out  as gdn_verify_span (ckpt is required)
 * Exactly one of `state` and `src` gives the initial state; with `src` the
 * span starts in place from the previous span's accepted checkpoint as in
 * gdn_verify_span_from (status, optional, counts requests whose node is out
 * of range; they write nothing). The conv state after the accepted position
 * comes from conv_state_advance. Errors: HRS_EINVAL, HRS_EALIGN,
 * HRS_EGEOMETRY, HRS_EUNSUPPORTED (W != 4, d_k/d_v outside the built set),
 * HRS_EDEVICE.
 */
int gdn_layer_verify_span(const hrs_gdn_layer_desc* desc, const void* x, const void* conv_w,
                          const void* conv_state, const void* a, const void* b,
                          const float* state, const hrs_span_source* src, float* ckpt,
                          float* out, int32_t* status, void* stream);

/* ------------------------------------------------------------------------ */
/* Causal depthwise conv1d over the span                                    */
/* ------------------------------------------------------------------------ */

typedef struct {
  int32_t n_req;     /* R                                                  */
  int32_t n_pos;     /* T                                                  */
  int32_t channels;  /* C, multiple of 8                                   */
  int32_t width;     /* W, conv width; 4 is built                          */
  hrs_dtype dtype;   /* dtype of x, w and the conv state                   */
  int32_t silu;      /* nonzero: y = z / (1 + exp(-z)) after the conv (to  */
                     /* a few ulp: hardware exp2 and reciprocal)           */
  hrs_topology topo;
  const int32_t* parent; /* host [n_req][n_pos] when topo == HRS_TREE      */
} hrs_conv_desc;

/*
 * conv1d_verify_span - causal depthwise conv over the span with the conv
 * state captured after every position ([P2] What Changed: the hybrid state
 * includes the conv state; [P1] Changes: conv state restored on device).
 *
 * For position t with parent p, the window is the parent's conv state
 * (conv_state for the root) followed by x_t, oldest first:
 *     y[r][t][c]        = sum_m w[c][m] window[m][c]     (float32 math)
 *     conv_ckpt[r][t]   = window[1..W-1]                 (exact copies)
 * w[c][W-1] multiplies the current input. No bias.
 *
 * Layouts:  x          [R][T][C]        dtype
 *           w          [C][W]           dtype
 *           conv_state [R][W-1][C]      dtype, oldest row first
 *           conv_ckpt  [R][T][W-1][C]   dtype
 *           y          [R][T][C]        float32
 * conv_ckpt == NULL: no capture, chain only; conv_state is advanced in
 * place to the state after the last position.
 * Errors: HRS_EINVAL, HRS_EALIGN, HRS_EGEOMETRY, HRS_EUNSUPPORTED (W != 4),
 * HRS_EDEVICE.
 */
int conv1d_verify_span(const hrs_conv_desc* desc, const void* x, const void* w,
                       void* conv_state, void* conv_ckpt, float* y, void* stream);

/*
 * conv1d_verify_span_nocapture - conv1d_verify_span that writes only y (chain
 * or tree); conv_state is read only and no per-position conv state is
 * written. With conv_state_advance below this replaces the [T][W-1][C] conv
 * checkpoint: the conv state after any position is the last W-1 entries of
 * [conv_state rows, x along that position's root path], so it can be rebuilt
 * from inputs the caller already holds.
 */
int conv1d_verify_span_nocapture(const hrs_conv_desc* desc, const void* x, const void* w,
                                 const void* conv_state, float* y, void* stream);

typedef struct {
  int32_t n_layers;  /* L */
  int32_t n_req;     /* R */
  int32_t n_pos;     /* T of the span just verified */
  int32_t channels;  /* C, multiple of 8 */
  int32_t width;     /* W; 4 is built */
  hrs_dtype dtype;   /* dtype of x and the conv state */
} hrs_conv_advance_desc;

/*
 * conv_state_advance - conv-state rollback without checkpoints: for every
 * layer l and request r, with n = accept_len[r] + 1 positions on the accepted
 * path path[r][0..n-1] (from accept_greedy),
 *     conv_state[l][r] = last W-1 rows of [conv_state[l][r], x[l][r][path[0]], ...,
 *                                          x[l][r][path[n-1]]]
 * in one launch, reading the index data on the device ([P1] Changes: conv
 * state restored on device). Bit-exact copies of input rows.
 * Layouts: x [L][R][T][C], conv_state [L][R][W-1][C] (dtype); path [R][T],
 * accept_len [R] int32 device. A request whose accept_len is outside [0, T)
 * or whose path holds an index outside [0, T) is left untouched; status
 * (optional device int32) receives the number of such requests.
 * Errors: HRS_EINVAL, HRS_EALIGN, HRS_EUNSUPPORTED (W != 4), HRS_EDEVICE.
 */
int conv_state_advance(const hrs_conv_advance_desc* desc, const void* x, void* conv_state,
                       const int32_t* path, const int32_t* accept_len, int32_t* status,
                       void* stream);

/* ------------------------------------------------------------------------ */
/* Greedy acceptance                                                        */
/* ------------------------------------------------------------------------ */

typedef struct {
  int32_t n_req;   /* R                                                    */
  int32_t n_pos;   /* T (rows of logits per request)                       */
  int32_t vocab;   /* V, multiple of 8                                     */
  hrs_dtype logit_dtype;
  hrs_topology topo;
  const int32_t* parent; /* host [n_req][n_pos] when topo == HRS_TREE      */
} hrs_accept_desc;

/* Bytes of device workspace accept_greedy needs for this descriptor
 * (0 if the descriptor is invalid). */
size_t accept_greedy_workspace_bytes(const hrs_accept_desc* desc);

/*
 * accept_greedy - greedy verification of one draft block per request
 * ([P2] Summary: greedy request whose output matches plain greedy decoding;
 * [P1] Verification: chain speculative generation and DDTree).
 *
 *  argmax[r][t]  = index of the largest logit of row (r, t); ties go to the
 *                  lowest index; NaN never wins; an all-NaN row gives 0.
 *  A position t >= 1 is matched when its parent is matched and
 *  tokens[r][t] == argmax[r][parent[t]]; the root (t = 0, the committed
 *  token) is always matched.
 *  accept_node[r] = the deepest matched position (lowest index on ties)
 *  accept_len[r]  = its depth = number of accepted drafts
 *  path[r][0..accept_len] = root .. accept_node, then -1 up to T
 *  bonus[r]       = argmax[r][accept_node], the next step's root token
 *
 * Layouts: logits [R][T][V] logit_dtype; tokens [R][T] int32; outputs int32
 * device arrays argmax [R][T], accept_node [R], accept_len [R],
 * path [R][T], bonus [R]. workspace: device scratch of at least
 * accept_greedy_workspace_bytes(desc) bytes, 16-byte aligned, contents
 * ignored on entry. Size limits: n_req * n_pos <= 65535 * 64 and
 * n_req * n_pos * ceil(V / 16384) <= 2^24 (else HRS_EINVAL). Errors:
 * HRS_EINVAL, HRS_EALIGN, HRS_EGEOMETRY, HRS_EDEVICE.
 */
int accept_greedy(const hrs_accept_desc* desc, const void* logits, const int32_t* tokens,
                  int32_t* argmax, int32_t* accept_node, int32_t* accept_len,
                  int32_t* path, int32_t* bonus, void* workspace,
                  size_t workspace_bytes, void* stream);

/* Largest workspace accept_greedy_noalloc can use: 1 MiB, the pass-1 keys of
 * up to 131,072 (row, 16384-logit chunk) pairs (e.g. 272 rows of 151,936
 * logits need 21,760 bytes). */
#define HRS_ACCEPT_NOALLOC_MAX_BYTES (1u << 20)

/*
 * accept_greedy_noalloc - accept_greedy for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation): the pass-1 keys live in a fixed device array of
 * HRS_ACCEPT_NOALLOC_MAX_BYTES inside the library instead of a caller's
 * workspace. The call itself allocates nothing. The array exists once per GPU
 * and stays for the life of the process; its device address is looked up on
 * the first call on each GPU (with that GPU current). Nothing in it needs to
 * start at zero: every key a call reads is written by the same call.
 * Calls that overlap in time on one GPU (different streams, or host threads
 * sharing a GPU) share the array and race; serialise them.
 * Arguments, results and errors as accept_greedy without the workspace,
 * plus HRS_EINVAL when accept_greedy_workspace_bytes(desc) exceeds
 * HRS_ACCEPT_NOALLOC_MAX_BYTES.
 */
int accept_greedy_noalloc(const hrs_accept_desc* desc, const void* logits, const int32_t* tokens,
                          int32_t* argmax, int32_t* accept_node, int32_t* accept_len, int32_t* path,
                          int32_t* bonus, void* stream);

/* ------------------------------------------------------------------------ */
/* On-device rollback                                                       */
/* ------------------------------------------------------------------------ */

typedef struct {
  int32_t n_layers;      /* L                                              */
  int32_t n_req;         /* R                                              */
  int32_t n_pos;         /* T                                              */
  int32_t n_vheads;      /* Hv                                             */
  int32_t d_k, d_v;
  int32_t conv_channels; /* C (0 with NULL conv buffers: no conv restore)  */
  int32_t conv_width;    /* W                                              */
  hrs_dtype conv_dtype;
} hrs_rollback_desc;

/*
 * rollback_restore - fast rollback: for every layer l and request r,
 *     state[l][r]      = ckpt[l][r][accept_node[r]]
 *     conv_state[l][r] = conv_ckpt[l][r][accept_node[r]]
 * in one launch, with the accepted index read from device memory, so no host
 * round trip sits between acceptance and restore ([P1] Changes: restore
 * split SSM and convolution state on device, synchronize once; [P3]
 * Summary: restore the accepted checkpoint without replay).
 *
 * Layouts:  ckpt       [L][R][T][Hv][d_v][d_k] float32
 *           state      [L][R][Hv][d_v][d_k]    float32
 *           conv_ckpt  [L][R][T][W-1][C]       conv_dtype (may be NULL)
 *           conv_state [L][R][W-1][C]          conv_dtype (NULL with conv_ckpt)
 *           accept_node [R] int32, device
 *           status     one int32, device: written by the launch with the
 *                      number of requests whose accept_node is outside
 *                      [0, T); those requests are left untouched.
 * Errors: HRS_EINVAL (also L * R > 65535, or one (layer, request) state or
 * conv state of 2 GiB or more), HRS_EALIGN, HRS_EDEVICE.
 */
int rollback_restore(const hrs_rollback_desc* desc, const float* ckpt, float* state,
                     const void* conv_ckpt, void* conv_state,
                     const int32_t* accept_node, int32_t* status, void* stream);

/* ------------------------------------------------------------------------ */
/* Feature ring                                                             */
/* ------------------------------------------------------------------------ */

typedef struct {
  int32_t ring_id;    /* which ring                                        */
  int32_t start_pos;  /* first slot, in [0, n_slots)                       */
  int32_t n_rows;     /* rows in the run, in [0, n_slots]                  */
  int32_t packed_row; /* first row in the packed buffer                    */
} hrs_ring_run;

typedef struct {
  int32_t n_rings;       /* rings (one per request)                        */
  int32_t n_slots;       /* S slots per ring                               */
  int32_t width;         /* D elements per row; D * elem_size % 16 == 0   */
  hrs_dtype dtype;
  int32_t n_packed_rows; /* rows in the packed buffer                      */
  int32_t n_runs;
  const hrs_ring_run* runs; /* host [n_runs]                               */
} hrs_ring_desc;

/*
 * ring_set_2d / ring_get_2d - batched feature-ring synchronisation: a run
 * of n rows starting at slot p occupies slots (p + i) mod S; a wrapping run
 * is split into two non-wrapping runs and every run of the call is copied by
 * one launch ([P1] Changes: one get_2d and one set_2d per non-wrapping run
 * instead of two transfers and a sync per token).
 *
 *   set: ring[id][(p + i) mod S][:] = packed[row + i][:]
 *   get: packed[row + i][:]         = ring[id][(p + i) mod S][:]
 * Layouts: ring [n_rings][S][D], packed [n_packed_rows][D], both dtype.
 * Destinations of one call must not overlap (set: ring slots; get: packed
 * rows), so the result never depends on copy order. Errors: HRS_EINVAL,
 * HRS_EALIGN, HRS_EDEVICE.
 */
int ring_set_2d(const hrs_ring_desc* desc, void* ring, const void* packed, void* stream);
int ring_get_2d(const hrs_ring_desc* desc, const void* ring, void* packed, void* stream);

/* ------------------------------------------------------------------------ */
/* Misc                                                                     */
/* ------------------------------------------------------------------------ */

/* Static description of a status code; never NULL. */
const char* hrs_strerror(int status);

/* HRS_ABI_VERSION of the built library. */
int hrs_abi_version(void);

/* hipError_t of the last launch an entry point made on the calling thread
 * (0 = success): the detail behind HRS_EDEVICE. Per-thread. */
int hrs_last_hip_error(void);

/* hipGetErrorString() of hrs_last_hip_error(); never NULL. */
const char* hrs_last_hip_error_string(void);

#ifdef __cplusplus
}
#endif

#endif /* HRS_H */
