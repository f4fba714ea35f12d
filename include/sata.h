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
  SATA_ERR_OOM = -5          /* host or device allocation failed in sata_build_basis */
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

/* Number of rows of order p: C(d_k + p - 1, p). */
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

/* Number of float32 values of one head's state: (d_v + 1) * C(d_k + P - 1, P - 1).
 * Layout: S as [D][d_v] row-major, then z as [D]; row order as in
 * sata_build_basis.  Row m holds unweighted monomials (the weights w_m are
 * applied on the query side).  Returns -1 on an invalid argument. */
int64_t sata_state_floats(const sata_basis* basis, int d_v);

/* Floats between consecutive heads' states in a state buffer: sata_state_floats
 * rounded up to a multiple of 64, so that every head starts 256-byte aligned.
 * A buffer of S states holds S * sata_state_stride floats; the values past
 * sata_state_floats in each head are padding that no call reads or writes.
 * Returns -1 on an invalid argument. */
int64_t sata_state_stride(const sata_basis* basis, int d_v);

/* Device workspace in bytes that sata_prefill needs for these sizes.  Long
 * sequences are processed in windows whose per-token records fit a cap of
 * 16 GiB; the environment variable SATA_PREFILL_WS_CAP (bytes, read at every
 * call: keep it unchanged between this query and the prefill) lowers or
 * raises it, trading workspace for one state reload per window. */
int sata_prefill_workspace(const sata_basis* basis, int B, int H, int n, int d_v, int dtype,
                           size_t* bytes);

/* Causal prefill of n tokens for B*H independent heads.
 *   q, k: [B, H, n, d_k], v: [B, H, n, d_v], contiguous, dtype as given,
 *         16-byte aligned.
 *   out:  [B, H, n, d_v] float32, 16-byte aligned; row i receives
 *         sum_{j<=i} T_P(q_i.k_j/c) v_j / sum_{j<=i} T_P(q_i.k_j/c), where the
 *         sum also runs over the tokens already folded into `state`.
 *   state:[B*H][sata_state_stride] float32, 16-byte aligned, in/out: the state
 *         of the tokens before this call (all zeros = empty prefix) is read and
 *         the state after the n tokens is written back.
 *   ws:   device workspace of at least sata_prefill_workspace bytes, 256-byte
 *         aligned; its contents on entry do not matter.
 * Arithmetic: float32 inputs run in fp32 throughout.  bfloat16 inputs run the
 * feature products and readout/update contractions on 16-bit MFMA operands
 * (f16 after exact per-head power-of-two scaling when the inputs' ranges
 * allow it, else bf16) with fp32 accumulation and an fp32 state; the tests
 * gate the row-normwise error against the exact truncated polynomial at 1e-5
 * (float32) and 3e-3 (bfloat16).  Heads whose query/key scales leave the
 * f16 range (query features beyond 2^12 after the scaling) use bf16 operands
 * and can exceed 3e-3 at small d_k over sequences of thousands of tokens.
 * n = 0 is a valid no-op. */
int sata_prefill(const sata_basis* basis, int B, int H, int n, int d_v, int dtype,
                 const void* q, const void* k, const void* v, float* out, float* state,
                 void* ws, size_t ws_bytes, void* stream);

/* Device workspace in bytes that sata_decode_step needs for S states. */
int sata_decode_workspace(const sata_basis* basis, int S, int d_v, int dtype, size_t* bytes);

/* One decode step for S independent states: each state takes one token
 * (q, k, v rows [S, d]), folds k and v into its state (S_m += phi_m(k) v,
 * z_m += phi_m(k)) and then reads out out = sum_m w_m phi_m(q) S_m /
 * sum_m w_m phi_m(q) z_m, so the new token attends to itself
 * [SATA page, "Engineering of constant compute cost"].
 *   q, k: [S, d_k]; v: [S, d_v] (dtype as given); out: [S, d_v] float32;
 *   state: [S][sata_state_stride] float32 in/out; 16-byte aligned out/state,
 *   256-byte aligned ws of at least sata_decode_workspace bytes.
 * S = 0 is a valid no-op. */
int sata_decode_step(const sata_basis* basis, int S, int d_v, int dtype, const void* q,
                     const void* k, const void* v, float* out, float* state, void* ws,
                     size_t ws_bytes, void* stream);

/* Static, human-readable name of a status code. */
const char* sata_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SATA_H */
