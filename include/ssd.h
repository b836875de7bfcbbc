/*
 * ssd.h -- C ABI of the MI355X (gfx950) SSD layer forward library, libssd.so.
 *
 * The operation is the forward pass of the SSD (structured state space duality)
 * layer, as defined on the page "Transformers are SSMs: Generalized Models and
 * Efficient Algorithms Through Structured State Space Duality" (paper summary):
 *   - section 2.4 / section 5.1: per head a scalar-identity SSM, A_t = a_t I,
 *     with head dimension P and state size N:
 *         h_t = a_t h_{t-1} + x_t B_t^T      (h_t is P x N)
 *         y_t = h_t C_t                      (y_t has P entries)
 *     equivalently Y = (L o C B^T) X with the 1-semiseparable mask
 *     L[i][j] = a_{j+1} ... a_i (i >= j), section 5.1;
 *   - section 6 and Listing 1: it is computed by the block (chunk)
 *     decomposition of that semiseparable matrix, with chunk length chunk_len;
 *   - section 7.2: heads are grouped, head h reads B and C of group h / (H/G);
 *   - section 8.3: a packed batch of variable-length sequences passes no state
 *     between sequences.
 * The result does not depend on chunk_len except through rounding.
 *
 * Conventions shared by every entry point:
 *   - All tensors are row-major and contiguous; "device" pointers are HIP device
 *     memory of the current device; every pointer must be 16-byte aligned.
 *   - a_t = exp(logA_t); logA is float32, finite and <= 0 (not checked: NaN or
 *     positive values propagate into the outputs).
 *   - The state before token 0 of a sequence is init_state (zeros when NULL); it
 *     is decayed by a_0.  final_state is the state after the last token.
 *   - The caller owns every buffer, including the workspace.  The library never
 *     allocates device memory, keeps no state between calls, never synchronizes,
 *     and enqueues all work on the given stream; results are valid once that
 *     stream reaches the enqueued work.  Calls with distinct workspaces may run
 *     concurrently.
 *   - Errors are returned as ssd_status codes; arguments are validated on the
 *     host before anything is enqueued, so a failing call enqueues nothing.
 *     Device-resident values (logA, seq_offsets contents) are not validated.
 */
#ifndef SSD_H
#define SSD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ssd_status {
    SSD_OK = 0,
    SSD_ERR_INVALID_ARG = -1,  /* null/misaligned/aliased pointer, bad dimension      */
    SSD_ERR_UNSUPPORTED = -2,  /* dtype, chunk_len, headdim or dstate outside support */
    SSD_ERR_WORKSPACE = -3,    /* workspace smaller than ssd_workspace_bytes()        */
    SSD_ERR_HIP = -4,          /* a HIP runtime call or kernel launch failed          */
    SSD_ERR_TOO_LARGE = -5     /* ssd_forward_noalloc: the problem needs more scratch
                                  than SSD_NOALLOC_SCRATCH_BYTES                      */
} ssd_status;

typedef enum ssd_dtype {
    SSD_DTYPE_F32 = 0,         /* X, B, C, Y in float32, fp32 MFMA                     */
    SSD_DTYPE_BF16 = 1         /* X, B, C, Y in bfloat16, bf16 MFMA, fp32 accumulation */
} ssd_dtype;

/* Problem description.
 *   batch     b  >= 1   rows of the batch (must be 1 when seq_offsets is given)
 *   seqlen    T  >= 1   tokens per batch row (total packed tokens with seq_offsets)
 *   nheads    H  >= 1
 *   headdim   P         multiple of 16, 16 <= P <= 256
 *   dstate    N         multiple of 16, 16 <= N <= 256
 *   ngroups   G  >= 1   H % G == 0
 *   chunk_len Q         one of 16, 32, 64, 128, 256 (the last chunk of a sequence
 *                       may be shorter)
 *   nseq                number of sequences: == batch without seq_offsets, else the
 *                       number of packed sequences (>= 1)
 *   dtype               an ssd_dtype value                                          */
typedef struct ssd_problem {
    int64_t batch;
    int64_t seqlen;
    int64_t nheads;
    int64_t headdim;
    int64_t dstate;
    int64_t ngroups;
    int64_t chunk_len;
    int64_t nseq;
    int32_t dtype;
    int32_t reserved;   /* must be 0 */
} ssd_problem;

/* Checks a problem description without touching any device.
 * Returns SSD_OK, SSD_ERR_INVALID_ARG (p NULL, a dimension out of range,
 * H % G != 0, nseq inconsistent) or SSD_ERR_UNSUPPORTED. */
int ssd_check_problem(const ssd_problem* p);

/* Device workspace in bytes that ssd_forward needs for this problem, or 0 when
 * ssd_check_problem(p) != SSD_OK.  Depends only on *p.  Host-only, no HIP call. */
size_t ssd_workspace_bytes(const ssd_problem* p);

/* The SSD forward pass (passages above).  Arguments, all device pointers unless noted:
 *   p            host pointer to the problem description
 *   X            [b, T, H, P]      dtype          input x
 *   logA         [b, T, H]         float32        log of the per-token, per-head decay a_t
 *   B            [b, T, G, N]      dtype          input projection B_t
 *   C            [b, T, G, N]      dtype          output projection C_t
 *   init_state   [nseq, H, P, N]   float32        state before token 0, or NULL for zeros
 *   seq_offsets  [nseq + 1]        int32          packed sequence boundaries, or NULL;
 *                                                 seq_offsets[0] = 0, seq_offsets[nseq] = T,
 *                                                 non-decreasing (empty sequences allowed:
 *                                                 their final state is their init state)
 *   Y            [b, T, H, P]      dtype (out)    y, rounded to dtype (round to nearest even)
 *   final_state  [nseq, H, P, N]   float32 (out)  state after the last token, or NULL to skip
 *   workspace    >= ssd_workspace_bytes(p) bytes of device scratch, 256-byte aligned
 *   hip_stream   hipStream_t to enqueue on (NULL = the default stream)
 * Y and final_state must not overlap any input or each other; the workspace (written by
 * the call) must overlap no input and no output.
 * Returns SSD_OK or an ssd_status error code (see the enum). */
int ssd_forward(const ssd_problem* p, const void* X, const float* logA, const void* B,
                const void* C, const float* init_state, const int32_t* seq_offsets, void* Y,
                float* final_state, void* workspace, size_t workspace_bytes, void* hip_stream);

/* One of the two launches that make up ssd_forward, with the same arguments and checks.
 *   stage 1: chunk cumsum of logA and the C B^T tiles of every chunk, written to the
 *            workspace (page section 6.1 and Listing 1 step 1 inputs); for the plans whose
 *            walk forms these itself (ssd_plan_describe: prep=none), the end state and
 *            total decay of every segment but the last of a sequence walked in segments,
 *            and each segment's entry state (section 6.2, Appendix B), or nothing
 *            (summary=none);
 *   stage 2: the chunk walk: outputs, chunk states and state passing (section 6.1 and
 *            6.2), reading the workspace that a stage-1 call with the same problem and
 *            inputs left there.
 * ssd_forward is stage 1 followed by stage 2 on the same stream.  This entry point is for
 * timing each launch on its own and for callers that place the two launches themselves.
 * Returns SSD_ERR_INVALID_ARG for a stage other than 1 or 2. */
int ssd_forward_stage(int stage, const ssd_problem* p, const void* X, const float* logA,
                      const void* B, const void* C, const float* init_state,
                      const int32_t* seq_offsets, void* Y, float* final_state, void* workspace,
                      size_t workspace_bytes, void* hip_stream);

/* One recurrent (decode) step for every sequence and head: the recurrence above for a
 * single token, continuing from a state a forward pass (final_state) or an earlier step
 * left (page section 2.4; the recurrent mode of section 3: constant memory and work per
 * token).  For each sequence s and head h with group g = h / (H/G):
 *     a = exp(logA[s, h]);  state[s, h] <- a state[s, h] + x[s, h] B[s, g]^T;
 *     y[s, h] = state[s, h] C[s, g]                 (after the update)
 * Problem: p->seqlen must be 1 and p->nseq == p->batch (one row per sequence);
 * headdim and dstate as for ssd_forward; chunk_len is not used.  Arguments (device):
 *   x      [b, H, P]     dtype          logA [b, H] float32
 *   B, C   [b, G, N]     dtype
 *   state  [b, H, P, N]  float32        read and overwritten in place
 *   y      [b, H, P]     dtype (out)    rounded to dtype (round to nearest even)
 * y and state must not overlap the inputs or each other.  No workspace.
 * Returns SSD_OK, SSD_ERR_INVALID_ARG, SSD_ERR_UNSUPPORTED or SSD_ERR_HIP. */
int ssd_decode_step(const ssd_problem* p, const void* x, const float* logA, const void* B,
                    const void* C, float* state, void* y, void* hip_stream);

/* Bytes of device scratch that ssd_backward needs for problem p (0 if p is invalid). */
size_t ssd_backward_workspace_bytes(const ssd_problem* p);

/* Gradients of the forward pass: for L = <dY, Y> + <dfinal, final_state>, the
 * derivatives of L with respect to X, logA, B, C and init_state.  The pages give only
 * the cost of training (section 6); the derivative is that of the recurrence of
 * section 2.4, the adjoint state G walked backwards over the tokens:
 *     G_t = a_{t+1} G_{t+1} + dy_t C_t^T        (G after the last token: dfinal)
 *     dx_t = G_t B_t,  dB_t = sum_h G_t^T x_t,  dC_t = sum_h S_t^T dy_t,
 *     dlogA_t = a_t <G_t, S_{t-1}>,  dinit = a_0 G_0       (sums over the group's heads)
 * computed as three forward passes on re-arranged operands (time reversed for dX, dinit
 * and dB) and small re-arranging and summing kernels.  The problem and the first six
 * arguments are those of the ssd_forward call being differentiated; further (device):
 *   Y            [b, T, H, P]     dtype          that call's output
 *   final_state  [nseq, H, P, N]  float32        its final state; required when dfinal
 *                                                is given, else may be NULL
 *   dY           [b, T, H, P]     dtype          gradient of the output
 *   dfinal       [nseq, H, P, N]  float32        gradient of the final state, or NULL (zero)
 *   dX           [b, T, H, P]     dtype (out)
 *   dlogA        [b, T, H]        float32 (out)
 *   dB, dC       [b, T, G, N]     dtype (out)
 *   dinit        [nseq, H, P, N]  float32 (out)  or NULL to skip (defined with or
 *                                                without init_state)
 *   workspace    >= ssd_backward_workspace_bytes(p) bytes, 256-byte aligned
 * The outputs must not overlap any input, the workspace or each other, and the workspace
 * overlaps no input.  Supported
 * problems: those of ssd_forward whose transposed problem (head dimension and state
 * size swapped) is supported too.  Returns SSD_OK or an ssd_status error code. */
int ssd_backward(const ssd_problem* p, const void* X, const float* logA, const void* B, const void* C,
                 const float* init_state, const int32_t* seq_offsets, const void* Y,
                 const float* final_state, const void* dY, const float* dfinal, void* dX, float* dlogA,
                 void* dB, void* dC, float* dinit, void* workspace, size_t workspace_bytes,
                 void* hip_stream);

/* Static English text for a status code (never NULL). */
const char* ssd_status_string(int status);

/* ABI revision of this header; bumped on any incompatible change. */
int ssd_abi_version(void);

/* The kernels ssd_forward launches for problem p, as text for logs and benchmarks:
 * "walk=<kernel>;prep=<kernel or none>;summary=<kernel or none>", for example
 * "walk=ssd_walk_fused_kernel<128, 5>;prep=none;summary=none".  Writes at most len
 * bytes, NUL-terminated, to buf (host memory).  Returns SSD_OK, the status of
 * ssd_check_problem for an invalid or unsupported problem, or SSD_ERR_INVALID_ARG for a
 * NULL buf or len 0.  No device work. */
int ssd_plan_describe(const ssd_problem* p, char* buf, size_t len);

/* ssd_forward for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  Same arguments, checks
 * and results as ssd_forward, without the workspace: the kernels that need scratch use a
 * fixed array of SSD_NOALLOC_SCRATCH_BYTES that the library holds on every device it runs
 * on until the process ends.  The call allocates nothing (no hipMalloc or allocating
 * library routine).  Its first call on a device looks up that device's array address; the
 * stream (NULL = the default stream) must belong to the current device.
 * All calls on one device share its array, and a call leaves its contents behind: calls
 * whose work overlaps on one device (on different streams, or from several threads) race
 * and give wrong results; calls ordered on one stream are safe.  Nothing in the array has
 * to start at zero.
 * Returns SSD_ERR_TOO_LARGE, before any device work, when ssd_workspace_bytes(p) exceeds
 * SSD_NOALLOC_SCRATCH_BYTES, else what ssd_forward returns. */
#define SSD_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int ssd_forward_noalloc(const ssd_problem* p, const void* X, const float* logA, const void* B,
                        const void* C, const float* init_state, const int32_t* seq_offsets,
                        void* Y, float* final_state, void* hip_stream);

#define SSD_ABI_VERSION 1

#ifdef __cplusplus
}
#endif

#endif /* SSD_H */
