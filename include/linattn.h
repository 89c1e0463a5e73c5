/*
 * linattn.h -- C ABI of liblinattn.so: linear attention with the elu(x)+1
 * feature map on AMD Instinct MI355X (gfx950).
 *
 * The operation ("Why Replace Attention? The Softmax Bottleneck and the Path
 * to Linear Time", §5.3, §6.2, §7.1, §7.2; "Transformers Are RNNs: Linear
 * Attention" knowledge note, "Reassociate the Products" and "Turn Causal
 * Attention into a Recurrence"):
 *
 *   phi(x) = elu(x) + 1  (x + 1 for x > 0, e^x otherwise), applied elementwise
 *   S_i = sum_{j in J(i)} phi(k_j) v_j^T   (C x M),   z_i = sum_{j in J(i)} phi(k_j)
 *   o_i = phi(q_i)^T S_i / phi(q_i)^T z_i
 *
 * with J(i) = {0..i} (causal, inclusive) or {0..N-1} (non-causal).  There is
 * no epsilon in the denominator.  In exact arithmetic phi > 0, so every
 * denominator is positive ("Why Replace Attention?", §5.4); in fp32 it can
 * underflow or overflow, the failure the "Transformers Are RNNs: Linear
 * Attention" knowledge note warns of under "Where It Breaks".
 *
 * Range.  o_i does not change when phi(q_i) is multiplied by a positive
 * constant, so the kernels scale each query row's phi(q_i) by an exact power
 * of two whenever its largest feature lies outside [-8, 65535] (the largest
 * scaled value then lies in [1, 2)); rows inside that interval are not
 * scaled, which changes no rounding.  Any finite query row is therefore
 * supported.  The supported range of keys and values is:
 *   every K feature >= -60, and N * (1 + max K) * max(1, max |V|) <= 2^100;
 * there outputs meet the library's accuracy (max |o - o_exact| / o_mag
 * <= 1e-4 for fp32 inputs, <= 2e-2 for bf16 inputs, with o_mag the same
 * weighted mean of |v|).  Below -60, accuracy degrades gradually.  When
 * every key feature that query i sees is below -104, e^x is 0 in fp32,
 * the denominator is exactly 0 and o_i is NaN (a decode step likewise,
 * while the state holds only such keys).  Inputs must be finite.
 *
 * Conventions shared by every entry point:
 *   - Pointers are device pointers (hipMalloc / PyTorch CUDA tensors) unless a
 *     comment says otherwise; all must be 16-byte aligned.  Kernels run on
 *     the calling thread's current HIP device: the buffers and `stream` must
 *     belong to it (this is not checked).
 *   - Tensors are contiguous row-major.  Q, K: [B, H, N, C]; V, O: [B, H, N, M].
 *   - This version supports C = M = 64 only (other values: LINATTN_ERR_SHAPE).
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls are
 *     asynchronous: they validate on the host, enqueue kernels on `stream` and
 *     return.  Device faults surface at the caller's next synchronisation.
 *   - Validation happens on the host before anything is enqueued; a call that
 *     returns an error has written no device memory.
 *   - The library allocates no device memory and keeps none between calls.
 *     Scratch space is the caller's `workspace`, except for
 *     linattn_forward_noalloc, whose scratch is a static device array that
 *     every device holds from load to process end.
 *   - The library is reentrant.  Its only global state is a per-thread error
 *     message, a per-device attribute cache, the per-device address of that
 *     static scratch, the segment-count override of linattn_set_segments and
 *     the optional kernel timer.
 *   - No C++ exception crosses this interface.
 */
#ifndef LINATTN_H
#define LINATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    LINATTN_OK = 0,
    LINATTN_ERR_NULL = 1,      /* a required pointer is NULL */
    LINATTN_ERR_SHAPE = 2,     /* negative size, C or M != 64, or a size that overflows */
    LINATTN_ERR_DTYPE = 3,     /* unknown element type */
    LINATTN_ERR_ALIGN = 4,     /* a pointer is not 16-byte aligned */
    LINATTN_ERR_ALIAS = 5,     /* an output overlaps an input */
    LINATTN_ERR_WORKSPACE = 6, /* workspace too small (or NULL while bytes are needed) */
    LINATTN_ERR_HIP = 7,       /* the HIP runtime reported an error at launch */
    LINATTN_ERR_ARG = 8        /* any other invalid argument */
} linattn_status;

typedef enum {
    LINATTN_F32 = 0,  /* IEEE binary32 */
    LINATTN_BF16 = 1  /* bfloat16; arithmetic is fp32 throughout */
} linattn_dtype;

/* Version of this interface (major * 10000 + minor * 100 + patch). */
int linattn_version(void);

/* Human-readable name of a status code (static string, never NULL). */
const char *linattn_status_string(linattn_status s);

/* Message describing the last error returned on the calling thread (static
 * per-thread buffer, never NULL; empty after a successful call). */
const char *linattn_last_error(void);

/* Bytes of device workspace `linattn_forward` needs for these arguments on the
 * current device (0 when the chosen plan needs none).  Returns 0 for invalid
 * arguments; `linattn_forward` reports those. */
size_t linattn_forward_workspace_bytes(int B, int H, int N, int C, int M, linattn_dtype dt, int causal);

/*
 * linattn_forward -- the chunked parallel forward over whole sequences.
 *
 *   causal != 0: o_i uses tokens j <= i ("Why Replace Attention?", §7.1; the
 *   causal prefix sums of §7.2 carried across chunks).
 *   causal == 0: o_i uses every token ("Why Replace Attention?", §6.2).
 *
 * Q, K: [B,H,N,C] in `dt`; V: [B,H,N,M] in `dt`; O: [B,H,N,M] in `dt`, written.
 * Accumulation is fp32; bf16 outputs are rounded to nearest-even.
 * workspace: device buffer of at least linattn_forward_workspace_bytes(...)
 *   bytes (may be NULL when that is 0).  Its contents on entry do not matter.
 * B == 0, H == 0 or N == 0: returns LINATTN_OK and enqueues nothing.
 * Errors: NULL (Q, K, V, O), SHAPE, DTYPE, ALIGN, ALIAS (O overlaps Q, K or
 *   V), WORKSPACE, HIP.
 * Results are deterministic: the same inputs, sizes and device give
 * bit-identical outputs.
 */
linattn_status linattn_forward(const void *Q, const void *K, const void *V, void *O, int B, int H, int N,
                               int C, int M, linattn_dtype dt, int causal, void *workspace,
                               size_t workspace_bytes, void *stream);

/*
 * linattn_forward_noalloc -- linattn_forward for callers that cannot allocate
 * device memory or pass a workspace: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  It allocates nothing: the
 * scratch space linattn_forward takes from `workspace` (the per-segment state
 * records) is a static device array of LINATTN_NOALLOC_SCRATCH_BYTES inside
 * the library, one per device, held until the process ends.
 *
 * Arguments and results as linattn_forward (bit-identical outputs), without
 * the workspace.  A problem whose plan needs more scratch than that
 * (linattn_forward_workspace_bytes(...) > LINATTN_NOALLOC_SCRATCH_BYTES)
 * returns LINATTN_ERR_WORKSPACE and enqueues nothing.  Every call on a device
 * shares that device's scratch: calls that overlap on one device (other
 * streams, other host threads) race and must be serialised by the caller.
 * The scratch needs no clearing between calls (every record is written
 * before it is read).  Errors otherwise as linattn_forward.
 */
#define LINATTN_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
linattn_status linattn_forward_noalloc(const void *Q, const void *K, const void *V, void *O, int B, int H, int N,
                                       int C, int M, linattn_dtype dt, int causal, void *stream);

/*
 * linattn_forward_state -- causal forward that starts from a given state and
 * returns the state after the last token: the prefill side of the handoff to
 * linattn_decode_step ("Transformers Are RNNs: Linear Attention" knowledge
 * note, "Putting It Together": only S_i and Z_i are carried forward; "[Paper
 * Review] Transformers are RNNs", §3.6: parallel in training, recurrent at
 * inference).
 *
 * S0: [B*H, C, M] fp32 and z0: [B*H, C] fp32, the state before token 0; both
 *   NULL means zero (S_0 = 0, z_0 = 0, "Why Replace Attention?", §7.2).  Both
 *   or neither must be given.
 * S_out: [B*H, C, M] fp32 and z_out: [B*H, C] fp32 receive S_N and z_N; both
 *   NULL skips the write.  Both or neither must be given.  They may be the
 *   same buffers as S0 / z0 (updated in place); they must not overlap Q, K,
 *   V or O.
 * Other arguments as linattn_forward with causal = 1.  With N == 0 the state
 *   is copied through (S_out = S0 or 0).
 */
linattn_status linattn_forward_state(const void *Q, const void *K, const void *V, void *O, int B, int H,
                                     int N, int C, int M, linattn_dtype dt, const float *S0, const float *z0,
                                     float *S_out, float *z_out, void *workspace, size_t workspace_bytes,
                                     void *stream);

/* Workspace for linattn_forward_state (the causal plan plus state staging). */
size_t linattn_forward_state_workspace_bytes(int B, int H, int N, int C, int M, linattn_dtype dt);

/* Bytes of device workspace `linattn_backward` needs (0 for invalid
 * arguments, which `linattn_backward` reports). */
size_t linattn_backward_workspace_bytes(int B, int H, int N, int C, int M, linattn_dtype dt, int causal);

/*
 * linattn_backward -- gradients of linattn_forward (zero initial state) with
 * respect to Q, K and V for a given dL/dO, in time and memory linear in N:
 * the gradients are themselves forward and reverse cumulative sums ("[Paper
 * Review] Transformers are RNNs", §3.5 "Gradient Computation"; "Transformers
 * Are RNNs: Linear Attention" knowledge note).  With g_i = dL/do_i,
 * den_i = phi(q_i)^T z_i, a_i = g_i / den_i and b_i = -(g_i . o_i) / den_i:
 *   dphi(q_i) = S_i a_i + b_i z_i            (S_i, z_i: prefix sums as in the forward)
 *   dphi(k_j) = R_j v_j + r_j,  dv_j = R_j^T phi(k_j)
 *   R_j = sum_{i: j in J(i)} phi(q_i) a_i^T,  r_j = sum_{i: j in J(i)} b_i phi(q_i)
 *   dq = dphi(q) * phi'(q),  phi'(x) = 1 for x > 0, e^x otherwise.
 * o_i is recomputed in fp32 (the forward's output is not an argument).
 * Range: the backward does not scale query rows, so on top of the forward's
 * range it needs every query row's largest feature in [-60, 2^30]; outside
 * it gradients may be NaN or inaccurate where the forward is not.
 *
 * Q, K, V, dO: [B,H,N,64] in `dt`; dQ, dK, dV: [B,H,N,64] in `dt`, written.
 * causal as in linattn_forward.  Accumulation is fp32; bf16 outputs are
 *   rounded to nearest-even.
 * workspace: device buffer of at least linattn_backward_workspace_bytes(...)
 *   bytes, 16-byte aligned; contents on entry do not matter.
 * B == 0, H == 0 or N == 0: returns LINATTN_OK and enqueues nothing.
 * Errors: NULL, SHAPE, DTYPE, ALIGN, ALIAS (an output overlaps an input, the
 *   outputs overlap each other, or the workspace overlaps any of them),
 *   WORKSPACE, HIP.  Deterministic like linattn_forward.
 */
linattn_status linattn_backward(const void *Q, const void *K, const void *V, const void *dO, void *dQ, void *dK,
                                void *dV, int B, int H, int N, int C, int M, linattn_dtype dt, int causal,
                                void *workspace, size_t workspace_bytes, void *stream);

/*
 * linattn_backward_after_forward -- linattn_backward for a workspace that
 * still holds what linattn_forward left in it: the per-segment (S, z)
 * records (segment totals, or with more than eight segments per head the
 * states at every segment start), which the backward then does not recompute
 * (saving a pass over K and V).
 *
 * Precondition (not checked): the last call that wrote `workspace` was
 * linattn_forward with the same Q, K, V contents, B, H, N, dt and causal
 * flag, on the same device and with the same segment override
 * (linattn_set_segments).  `workspace` must hold
 * linattn_backward_workspace_bytes(...) bytes; linattn_forward uses only its
 * first linattn_forward_workspace_bytes(...).  With a violated precondition
 * the gradients are wrong; nothing faults.  Other arguments, errors and
 * results as linattn_backward (the results are bit-identical).
 */
linattn_status linattn_backward_after_forward(const void *Q, const void *K, const void *V, const void *dO, void *dQ,
                                              void *dK, void *dV, int B, int H, int N, int C, int M,
                                              linattn_dtype dt, int causal, void *workspace, size_t workspace_bytes,
                                              void *stream);

/* Bytes of device workspace the pair linattn_forward_train /
 * linattn_backward_train needs (0 for invalid arguments).  At least
 * linattn_backward_workspace_bytes(...). */
size_t linattn_train_workspace_bytes(int B, int H, int N, int C, int M, linattn_dtype dt, int causal);

/*
 * linattn_forward_train -- linattn_forward for a training step: the same
 * outputs, bit for bit, and it also leaves in `workspace` what
 * linattn_backward_train reads: the per-segment (S, z) records and, for bf16
 * causal calls, 1/den_i of every token (den_i = phi(q_i)^T z_i, the
 * normaliser of "Why Replace Attention?", §5.4), 4 bytes per token.
 *
 * workspace: device buffer of at least linattn_train_workspace_bytes(...)
 *   bytes, 16-byte aligned, disjoint from Q, K, V and O.
 * Other arguments and errors as linattn_forward.
 */
linattn_status linattn_forward_train(const void *Q, const void *K, const void *V, void *O, int B, int H, int N,
                                     int C, int M, linattn_dtype dt, int causal, void *workspace,
                                     size_t workspace_bytes, void *stream);

/*
 * linattn_backward_train -- the gradients of linattn_backward after
 * linattn_forward_train, reading that forward's output O and saved 1/den_i.
 * The gradients are the forward and reverse cumulative sums of
 * "[Paper Review] Transformers are RNNs", §3.5 ("Gradient Computation").
 *
 * bf16, causal: with O and 1/den_i the per-token factors a_i = g_i / den_i
 *   and b_i = -(g_i . o_i) / den_i need no state, so one pass over Q, dO and
 *   O forms the reverse sums and one left-to-right pass over Q, K, V and dO
 *   writes dQ, dK and dV together (10 tensor passes of B*H*N*64 elements in
 *   all, against 13 for linattn_backward_after_forward).  b_i is formed from
 *   the stored (bf16) O, so the results differ from linattn_backward's in
 *   rounding only; the error bounds of linattn_backward hold.
 * fp32, or causal = 0: linattn_backward_after_forward on the records the
 *   forward left (bit-identical to linattn_backward); O is checked, not read.
 *
 * O: [B,H,N,64] in `dt`, the output of that linattn_forward_train call;
 *   16-byte aligned; must not overlap dQ, dK, dV or the workspace.
 * Precondition (not checked): the last call that wrote `workspace` was
 * linattn_forward_train with the same Q, K, V contents, B, H, N, dt and
 * causal flag, on the same device and segment override, and O is unchanged
 * since.  With a violated precondition the gradients are wrong; nothing
 * faults.
 * Other arguments, errors and results as linattn_backward (ALIAS also when O
 *   overlaps an output or the workspace).  Deterministic.
 */
linattn_status linattn_backward_train(const void *Q, const void *K, const void *V, const void *O, const void *dO,
                                      void *dQ, void *dK, void *dV, int B, int H, int N, int C, int M,
                                      linattn_dtype dt, int causal, void *workspace, size_t workspace_bytes,
                                      void *stream);

/*
 * linattn_decode_step -- one constant-state recurrent step for BH independent
 * heads ("Why Replace Attention?", §7.2, steps 1-4; §7.4 constant work per
 * step):
 *   S += phi(k) v^T;  z += phi(k);  o = phi(q)^T S / phi(q)^T z   (read after update)
 *
 * S: [BH, C, M] fp32, S[h][c][m], read and updated in place.
 * z: [BH, C] fp32, read and updated in place.
 * q, k: [BH, C] in `dt`; v: [BH, M] in `dt`.  o: [BH, M] fp32, written.
 * A fresh sequence starts from S = 0, z = 0 (caller clears them).
 * BH == 0: LINATTN_OK, nothing enqueued.
 * Errors: NULL, SHAPE, DTYPE, ALIGN, ALIAS (o overlaps S or z, or S overlaps
 *   z, or q/k/v overlap S, z or o), HIP.
 */
linattn_status linattn_decode_step(float *S, float *z, const void *q, const void *k, const void *v, float *o,
                                   int BH, int C, int M, linattn_dtype dt, void *stream);

/*
 * linattn_decode_step_strided -- linattn_decode_step with the q, k and v
 * vectors of consecutive heads `row_stride` elements apart instead of 64, so
 * that they can be column slices of one projection output: with a q/k/v
 * projection whose columns are ordered (head, {q, k, v}, 64), q = out,
 * k = out + 64, v = out + 128 and row_stride = 192.
 *
 * row_stride: >= 64, and row_stride * element size a multiple of 16 bytes.
 * q, k, v: head h's vector at q + h * row_stride (likewise k, v), in `dt`;
 *   they may overlap each other, but not S, z or o.
 * Other arguments, layouts and errors as linattn_decode_step (SHAPE for a
 * bad stride, ALIGN for a misaligned one).
 */
linattn_status linattn_decode_step_strided(float *S, float *z, const void *q, const void *k, const void *v, float *o,
                                           int BH, int C, int M, linattn_dtype dt, long long row_stride,
                                           void *stream);

/*
 * Kernel timer (measurement support).  When enabled, the library brackets
 * each kernel it launches with HIP events recorded on the launch stream and,
 * when linattn_timer_read() is called, adds up the elapsed times per kernel
 * name.  Reading synchronises with the recorded events.  Off by default;
 * enabling it adds two event records per kernel.
 */
void linattn_timer_enable(int on);
void linattn_timer_reset(void);
/* Total milliseconds and launch count recorded for `kernel` (a name printed
 * by linattn_timer_names).  Returns 0 if found, -1 otherwise. */
int linattn_timer_read(const char *kernel, double *total_ms, long *launches);
/* Writes the ';'-separated kernel names seen so far into buf (NUL-terminated,
 * truncated to len).  Returns the full length needed. */
size_t linattn_timer_names(char *buf, size_t len);

/*
 * Plan override (measurement support): forces the number of sequence
 * segments per head used by linattn_forward (0 restores the automatic
 * choice).  Returns the previous override.  Applies to subsequent calls
 * process-wide.  Any value gives the same result up to fp32 rounding order.
 */
int linattn_set_segments(int segments_per_head);

/* Segments per head the planner picks for these arguments (after override). */
int linattn_plan_segments(int B, int H, int N, linattn_dtype dt, int causal);

#ifdef __cplusplus
}
#endif

#endif /* LINATTN_H */
