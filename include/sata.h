/*
 * sata.h -- C ABI of the MI355X (gfx950) library for causal symmetry-aware
 * Taylor-approximated softmax attention (SATA).
 *
 * The method (SATA summary page, blog.hotdry.top, "symmetry-aware Taylor
 * approximation": sections "Core insight: symmetric tensor decomposition" and
 * "Engineering of constant compute cost"): exp(q.k/c) is replaced by its Taylor
 * polynomial of orders 0..P-1, and every power (q.k)^p is factored through the
 * minimal basis of the order-p symmetric tensor -- the multisets
 * i1 <= ... <= ip over [0, d_k) -- so that a head keeps a fixed-size causal
 * state of (d_v + 1) * C(d_k + P - 1, P - 1) values:
 *     S_m = sum_j phi_m(k_j) v_j,   z_m = sum_j phi_m(k_j),
 *     out_i = sum_m w_m phi_m(q_i) S_m / sum_m w_m phi_m(q_i) z_m,
 * where phi_m(x) = prod_r x[i_r] and w_m = mult(m) / (p! c^p) with
 * mult(m) = p! / prod(count!) the number of index tuples the multiset stands for.
 * The sum over j includes the current token (j <= i).
 *
 * Conventions shared by every call:
 *   - All device pointers are HIP device memory on the device the basis was
 *     built on, allocated and owned by the caller.  The library owns only the
 *     basis handle (host tables plus a device copy) until sata_free_basis.
 *   - Hot calls (sata_prefill, sata_decode_step) are asynchronous on `stream`
 *     (a hipStream_t passed as void*, NULL = the default stream).  They never
 *     allocate, never synchronise and never free.
 *   - Every argument is checked on the host before any launch.  A call that
 *     returns an error other than SATA_ERR_HIP has launched nothing and
 *     changed no buffer.  SATA_ERR_HIP reports a launch failure.
 *   - No exceptions cross the ABI.  sata_status_string names every status.
 *   - A basis may be shared by several threads and streams; one state buffer
 *     must not be used by two calls in flight at once.
 *   - Supported: d_k = d_v in {8, 16, 32, 64}, P in {1, 2, 3, 4, 5}, c > 0 finite.
 *     Inputs are float32 or bfloat16; state and outputs are float32.
 */
#ifndef SATA_H
#define SATA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct sata_basis sata_basis; /* opaque, immutable after build */

enum sata_status {
  SATA_OK = 0,
  SATA_ERR_INVALID_ARG = -1, /* null / misaligned pointer, negative size, bad dtype, wrong device */
  SATA_ERR_UNSUPPORTED = -2, /* d_k, d_v or P outside the compiled instances */
  SATA_ERR_WORKSPACE = -3,   /* ws too small (or null while bytes > 0) */
  SATA_ERR_HIP = -4,         /* a HIP runtime call or kernel launch failed */
  SATA_ERR_OOM = -5,         /* host or device allocation failed in sata_build_basis */
  SATA_ERR_SCRATCH = -6      /* sata_decode_step_noalloc: the call needs more than its static scratch */
};

enum sata_dtype { SATA_F32 = 0, SATA_BF16 = 1 }; /* input dtype of q, k, v */

/* Build the minimal-basis and coefficient tables for (d_k, P, c) on the host,
 * then upload them to the current HIP device (synchronous).  For each order
 * p = 0..P-1 the rows are the multisets i1 <= ... <= ip over [0, d_k) in
 * lexicographic order; orders are concatenated by ascending p (order 0 is one
 * empty multiset), so the total is C(d_k + P - 1, P - 1)  [SATA page, "Core
 * insight: symmetric tensor decomposition" and "Engineering of constant
 * compute cost"].  On success *out holds a handle to free with sata_free_basis. */
int sata_build_basis(int d_k, int P, double c, sata_basis** out);

/* The same tables, built on the host only (no HIP call, no device copy).
 * Such a handle answers every query below except sata_basis_download_rows,
 * and the compute calls reject it with SATA_ERR_INVALID_ARG. */
int sata_build_basis_host(int d_k, int P, double c, sata_basis** out);

/* Release the handle and its device tables.  NULL is accepted. */
void sata_free_basis(sata_basis* basis);

/* Basic facts of a handle. */
int sata_basis_info(const sata_basis* basis, int* d_k, int* P, double* c, int64_t* total_rows);

/* Number of rows of order p: C(d_k + p - 1, p), the size of the minimal basis
 * of the order-p symmetric tensor [SATA page, "Core insight: symmetric tensor
 * decomposition"]; summed over p = 0..P-1 it is C(d_k + P - 1, P - 1)
 * [same page, "Engineering of constant compute cost"].  *rows is written on
 * success; SATA_ERR_INVALID_ARG for a null handle or pointer or p outside
 * [0, P). */
int sata_basis_rows(const sata_basis* basis, int p, int64_t* rows);

/* Copy the host tables of order p: idx [rows * p] int32 (row-major, 0-based,
 * i1 <= ... <= ip) and mult [rows] uint32 (p!/prod(count!)).  Either pointer
 * may be NULL to skip it. */
int sata_basis_copy_tables(const sata_basis* basis, int p, int32_t* idx, uint32_t* mult);

/* Download the device copy of the row table used by the kernels, for every
 * row r in order: packed[r] = i1 | i2 << 6 | i3 << 12 | i4 << 18 | p << 24
 * (six bits per index, unused indices zero) and weight[r] =
 * float(mult / (p! c^p)).  Host pointers of total_rows elements; synchronous. */
int sata_basis_download_rows(const sata_basis* basis, uint32_t* packed, float* weight);

/* Number of float32 values of one head's state: (d_v + 1) * C(d_k + P - 1, P - 1),
 * the fixed state size of the SATA page, section "Engineering of constant
 * compute cost" (S_p holds d_v columns and z_p one per basis row; it does not
 * depend on the sequence length).
 * Layout: S as [D][d_v] row-major, then z as [D]; row order as in
 * sata_build_basis.  Row m holds unweighted monomials (the weights w_m are
 * applied on the query side).  Returns -1 on a null handle or d_v != d_k. */
int64_t sata_state_floats(const sata_basis* basis, int d_v);

/* A head stride (floats) for the *_strided calls: sata_state_floats rounded
 * up to a multiple of 64, so that every head starts 256-byte aligned and the
 * decode step streams its rows with 16-byte accesses (the fastest layout).
 * The values past sata_state_floats in each head are padding that no call
 * reads or writes.  Returns -1 on a null handle or d_v != d_k. */
int64_t sata_state_stride(const sata_basis* basis, int d_v);

/* Device workspace in bytes for sata_prefill at these sizes.  A prefill runs
 * its heads in groups and each group's tokens in call windows (multiples of
 * 512 tokens for bfloat16 inputs); the workspace holds the records of one
 * group and window.  With bfloat16 inputs, one length for every head and
 * too few heads to fill the chip, each head instead runs as parallel
 * sequence segments [SATA page, "Engineering of constant compute cost": the
 * state is a sum over the keys, so it composes over token ranges]: a
 * state-only pass over all but the last segment, a prefix sum of the segment
 * states, then every segment in full from its prefix state; the workspace
 * then also holds one state per segment.  The environment variable
 * SATA_PREFILL_SEGMENTS=0 (read at every call, like the cap below) turns
 * segments off.  The call picks, from the workspace it is given, the cut
 * of least modelled time that fits: more, smaller groups cost little while
 * each group still fills the chip's 256 compute units, while every extra
 * window reloads the state once.  The size returned here is that of the
 * smallest cut within 2 % of the least modelled time whose groups still fill
 * the chip (256 heads of 4096 tokens at d = 64, P = 4: 2.5 GB where a single
 * group needs 14.8 GB, measured as fast); a larger workspace selects the
 * least-time cut, a smaller one (down to sata_prefill_workspace(basis, 1, 1,
 * min(n, 512), ...) bytes, which always works) a slower one.  All sizes are
 * capped at 16 GiB, or at the byte count in the environment variable
 * SATA_PREFILL_WS_CAP (read at every call: keep it unchanged between this
 * query and the prefill).  SATA_ERR_WORKSPACE when the cap is below that
 * minimum. */
int sata_prefill_workspace(const sata_basis* basis, int B, int H, int n, int d_v, int dtype,
                           size_t* bytes);

/* Causal prefill of n tokens for B*H independent heads [SATA page, "Engineering
 * of constant compute cost": each key enters the fixed-size state
 * S_m += phi_m(k) v, z_m += phi_m(k), and each query reads it out through the
 * weighted feature map; the sum over j runs to the current token].
 *   q, k: [B, H, n, d_k], v: [B, H, n, d_v], contiguous, dtype as given,
 *         16-byte aligned.
 *   out:  [B, H, n, d_v] float32, 16-byte aligned; row i receives
 *         sum_{j<=i} T_P(q_i.k_j/c) v_j / sum_{j<=i} T_P(q_i.k_j/c), where the
 *         sum also runs over the tokens already folded into `state`.
 *   state:[B*H][sata_state_floats] float32 (heads packed back to back),
 *         4-byte aligned, in/out: the state of the tokens before this call
 *         (all zeros = empty prefix) is read and the state after the n tokens
 *         is written back.  Nothing outside B*H*sata_state_floats floats is
 *         touched.
 *   ws:   device workspace of ws_bytes bytes, 256-byte aligned: at least
 *         the one-head, one-window minimum given at sata_prefill_workspace
 *         (whose returned size is the default); its contents on entry do
 *         not matter.
 * Arithmetic: float32 inputs run in fp32 throughout.  bfloat16 inputs run the
 * feature products and readout/update contractions on 16-bit MFMA operands
 * (f16 after exact per-head power-of-two scaling when the inputs' ranges
 * allow it, else bf16) with fp32 accumulation and an fp32 state; the tests
 * gate the row-normwise error against the exact truncated polynomial at 1e-5
 * (float32) and 3e-3 (bfloat16), on both operand paths.
 * Errors: SATA_ERR_INVALID_ARG (null or misaligned pointer, B, H < 1, n < 0,
 * bad dtype, a basis of another device or a host-only basis),
 * SATA_ERR_UNSUPPORTED (d_v != d_k, B*H > 65535), SATA_ERR_WORKSPACE.
 * n = 0 is a valid no-op. */
int sata_prefill(const sata_basis* basis, int B, int H, int n, int d_v, int dtype,
                 const void* q, const void* k, const void* v, float* out, float* state,
                 void* ws, size_t ws_bytes, void* stream);

/* sata_prefill with heads state_stride floats apart in `state`
 * (state_stride >= sata_state_floats, else SATA_ERR_INVALID_ARG); the floats
 * between sata_state_floats and state_stride of each head are not touched.
 * sata_state_stride gives the aligned stride the decode step streams
 * fastest. */
int sata_prefill_strided(const sata_basis* basis, int B, int H, int n, int d_v, int dtype,
                         const void* q, const void* k, const void* v, float* out, float* state,
                         int64_t state_stride, void* ws, size_t ws_bytes, void* stream);

/* Prefill with a length per head [SATA page, "Engineering of constant
 * compute cost": the state has the same size whatever a sequence's length, so
 * sequences of different lengths batch uniformly]: head h (= b * H + h' in
 * [B, H] order) takes only its first lengths[h] tokens of the n slots of
 * q, k, v; each of them attends causally to the head's earlier tokens (and
 * its state), exactly as in sata_prefill_strided over that head alone.  The
 * state absorbs exactly lengths[h] tokens; output rows past lengths[h] are
 * written as zeros.  lengths: [B*H] int32 in device memory (read by the
 * kernels, so the host cannot check it: values are clamped to [0, n]).  A
 * length of 1 on a head with a state is one decode step, so one call serves
 * a batch that mixes prefill chunks and decode steps.  Other arguments and
 * errors as for sata_prefill_strided; the workspace is sata_prefill_workspace
 * for (B, H, n). */
int sata_prefill_varlen(const sata_basis* basis, int B, int H, int n, int d_v, int dtype,
                        const void* q, const void* k, const void* v, const int32_t* lengths,
                        float* out, float* state, int64_t state_stride, void* ws, size_t ws_bytes,
                        void* stream);

/* Device workspace in bytes that sata_decode_step needs for S states. */
int sata_decode_workspace(const sata_basis* basis, int S, int d_v, int dtype, size_t* bytes);

/* One decode step for S independent states: each state takes one token
 * (q, k, v rows [S, d]), folds k and v into its state (S_m += phi_m(k) v,
 * z_m += phi_m(k)) and then reads out out = sum_m w_m phi_m(q) S_m /
 * sum_m w_m phi_m(q) z_m, so the new token attends to itself
 * [SATA page, "Engineering of constant compute cost"].
 *   q, k: [S, d_k]; v: [S, d_v] (dtype as given); out: [S, d_v] float32,
 *   16-byte aligned; state: [S][sata_state_floats] float32 in/out (packed,
 *   4-byte aligned); ws: 256-byte aligned, at least sata_decode_workspace
 *   bytes.  Errors as for sata_prefill.
 * S = 0 is a valid no-op. */
int sata_decode_step(const sata_basis* basis, int S, int d_v, int dtype, const void* q,
                     const void* k, const void* v, float* out, float* state, void* ws,
                     size_t ws_bytes, void* stream);

/* sata_decode_step with states state_stride floats apart (state_stride >=
 * sata_state_floats).  With a stride that is a multiple of 4 floats and a
 * 16-byte aligned state (sata_state_stride), rows stream as 16-byte
 * accesses; otherwise as 4-byte ones. */
int sata_decode_step_strided(const sata_basis* basis, int S, int d_v, int dtype, const void* q,
                             const void* k, const void* v, float* out, float* state,
                             int64_t state_stride, void* ws, size_t ws_bytes, void* stream);

/* ---- Mixed-precision decode state ------------------------------------------
 * A second state format for the memory-bound decode step [SATA page,
 * "Precision/efficiency trade-off parameter" (the P = 4 error is of the order
 * of Float16 precision) and "Hardware optimisation path and current
 * limitations" (a Float16 state roughly halves the bandwidth)]: rows of
 * orders 0 and 1 of S and all of z stay float32; rows of order >= 2 of S are
 * stored as float16, in tiles of rows that each carry one power-of-two scale,
 * re-chosen by the decode step whenever it writes the tile back so that a
 * growing state cannot overflow.  At d_k = 64, P = 4 a state is 6.33 MB
 * instead of 12.46 MB.  The layout inside a state is private to the library;
 * states are sata_mixed_state_bytes apart (a multiple of 256) in a 256-byte
 * aligned buffer.  A prefill runs on the float32 state; sata_state_to_mixed
 * hands it to the decode format, sata_state_from_mixed hands it back (for a
 * continuation prefill).  Errors as for sata_decode_step. */

/* Bytes of one mixed state (-1 on a null handle or d_v != d_k). */
int64_t sata_mixed_state_bytes(const sata_basis* basis, int d_v);

/* S float32 states ([S][state_stride] floats) -> S mixed states. */
int sata_state_to_mixed(const sata_basis* basis, int S, int d_v, const float* state, int64_t state_stride,
                        void* mixed, void* stream);

/* S mixed states -> S float32 states ([S][state_stride] floats). */
int sata_state_from_mixed(const sata_basis* basis, int S, int d_v, const void* mixed, float* state,
                          int64_t state_stride, void* stream);

/* Device workspace in bytes that sata_decode_step_mixed needs for S states. */
int sata_decode_mixed_workspace(const sata_basis* basis, int S, int d_v, int dtype, size_t* bytes);

/* sata_decode_step on S mixed states: the same update and readout, the
 * float16 rows read, updated and read out in float32 and rounded (to nearest
 * even, after their tile's scale) when written back. */
int sata_decode_step_mixed(const sata_basis* basis, int S, int d_v, int dtype, const void* q,
                           const void* k, const void* v, float* out, void* mixed, void* ws,
                           size_t ws_bytes, void* stream);

/* ---- Exact causal softmax attention (the baseline) -------------------------
 * out_i = sum_{j<=i} exp(q_i.k_j/c) v_j / sum_{j<=i} exp(q_i.k_j/c), computed
 * stably with a running maximum [MoA page, section "DNF derivation"]; its
 * per-token work grows with the position [SATA page, "Scale bottleneck of
 * conventional self-attention": n (2 d_k + 2 d_v + 3) FLOPs at position n],
 * which SATA's fixed-size state avoids.  It is here to measure that
 * crossover on this hardware, not as part of the SATA path.
 *   q, k, v: [B, H, n, d] contiguous (float32 or bfloat16), out: [B, H, n, d]
 *   float32, all 16-byte aligned; d in {8, 16, 32, 64}; c > 0.  No basis and
 *   no workspace.  bfloat16: scores and value sums on bf16 MFMA with fp32
 *   accumulation, the probabilities as two bf16 parts; float32: fp32
 *   arithmetic throughout.  Asynchronous on `stream`. */
int sata_softmax_attention(int B, int H, int n, int d, int dtype, double c, const void* q, const void* k,
                           const void* v, float* out, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * sata_decode_step_strided without a workspace argument.  The per-tile
 * partial records live in a file-scope device array of
 * sata_decode_noalloc_max_bytes() bytes (32 MiB), one per device, held until
 * the process ends and resolved once per device when a basis is built there.
 * A call whose sata_decode_workspace exceeds that size returns
 * SATA_ERR_SCRATCH (at d = 64, P = 4: up to 81 states a call with bf16
 * inputs, 43 with fp32 inputs) and launches
 * nothing.  The call itself allocates and frees nothing.  Every call on one
 * device shares that device's array: calls that overlap in time on one
 * device (other streams, other threads) race and must be serialised by the
 * caller.  Each call overwrites every record it reads, so nothing needs
 * clearing between calls.  Results are bit-identical to sata_decode_step_strided. */
int sata_decode_step_noalloc(const sata_basis* basis, int S, int d_v, int dtype, const void* q,
                             const void* k, const void* v, float* out, float* state,
                             int64_t state_stride, void* stream);

/* Bytes of the static scratch array behind sata_decode_step_noalloc. */
size_t sata_decode_noalloc_max_bytes(void);

/* Static, human-readable name of a status code. */
const char* sata_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SATA_H */
