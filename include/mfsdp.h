/*
 * mfsdp.h -- C ABI of the owner-local optimizer step on MI355X (gfx950).
 *
 * Source of the operations: "MatrixFSDP: communication-free matrix optimizers
 * under ZeRO-3 parameter sharding" (arxivlens page, Abstract; gist.science
 * technical summaries, section "Methodologie", part 1 "owner-shaped
 * placement").  Under owner-shaped ZeRO-3 placement every 2D weight lives whole
 * on one data-parallel owner and every other rank holds an empty shard for it;
 * after the ordinary gradient reduction the owner holds the whole gradient, so
 * its Muon step -- momentum, Newton-Schulz orthogonalization of the whole
 * matrix, update -- involves no communication.  Tensors that are not 2D
 * matrices are gathered on tail owners and updated there with AdamW.  This
 * library is that step on one GPU:
 *
 *   mfsdp_muon_step   -- Muon on the owner's list of whole matrices,
 *   mfsdp_adamw_tail  -- AdamW on a packed fp32 tail buffer.
 *
 * Conventions shared by every entry point
 *   - Every pointer named "device" is a device (HBM) address on the current
 *     HIP device.  The caller owns every buffer; the library never allocates
 *     or frees device memory.  Host pointers are read only during the call.
 *   - Work is enqueued asynchronously on `stream`; no call waits for device
 *     work to finish.
 *   - All arguments are validated before anything is enqueued.  On any
 *     status other than MFSDP_OK nothing has been modified, except for
 *     MFSDP_ERR_HIP, which is returned when the HIP runtime fails after work
 *     was enqueued (the contents of the outputs are then undefined).
 *   - mfsdp_last_error() returns a thread-local description of the last
 *     failure on the calling thread.  No C++ exception crosses this ABI.
 *   - Non-finite inputs are not checked: they propagate to the outputs.
 */
#ifndef MFSDP_H_
#define MFSDP_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mfsdp_status {
  MFSDP_OK = 0,
  MFSDP_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size, bad scalar    */
  MFSDP_ERR_UNSUPPORTED = 2,      /* dtype or size this build cannot run   */
  MFSDP_ERR_WORKSPACE = 3,        /* workspace too small or misaligned     */
  MFSDP_ERR_ALIAS = 4,            /* two buffers that must not overlap do  */
  MFSDP_ERR_HIP = 5               /* the HIP runtime reported an error     */
} mfsdp_status_t;

typedef enum mfsdp_dtype {
  MFSDP_DTYPE_F32 = 0,  /* W, G, M and the Newton-Schulz iterates in fp32    */
  MFSDP_DTYPE_BF16 = 1  /* W, G, M in bf16; NS iterates bf16, fp32 accumulate */
} mfsdp_dtype_t;

/* Additive guard of the Frobenius normalization X0 = U / (||U||_F + eps). */
#define MFSDP_NS_EPS 1e-7f

/* Byte alignment required of every device buffer and of the workspace. */
#define MFSDP_ALIGNMENT 16

/*
 * One whole matrix owned by this rank (arxivlens Abstract: the owner holds the
 * complete 2D weight; its gradient arrives whole after the backward
 * reduction).  Stored row-major as rows x cols (rows = out_features),
 * contiguous, in the call's dtype.
 *
 *   weight      device, rows*cols, updated in place:
 *                 W <- (1 - lr*weight_decay) * W - lr * scale * O
 *   grad        device, rows*cols, read only
 *   momentum    device, rows*cols, updated in place: M <- beta*M + G
 *   update_out  device fp32 rows*cols, or NULL.  When given it receives O, the
 *               orthogonalized update before lr and scale.
 *   scale       the per-matrix update scale s (> 0, finite).  The common
 *               convention is sqrt(max(1, rows/cols)); the pages fix none.
 */
typedef struct mfsdp_matrix {
  void* weight;
  const void* grad;
  void* momentum;
  float* update_out;
  int64_t rows;
  int64_t cols;
  float scale;
} mfsdp_matrix_t;

/*
 * Workspace bytes that mfsdp_muon_step needs for this list (host call, no
 * device access).  The workspace holds the Newton-Schulz iterates of every
 * matrix (two m_pad x n_pad buffers and two m_pad x m_pad buffers per matrix,
 * m = min(rows, cols), n = max(rows, cols), padded to the 256-wide tile), the
 * per-block partial sums of the Frobenius norm and the launch descriptors.
 * Only rows, cols are read from `mats`.  n_mats == 0 gives 0 bytes.
 * Errors: MFSDP_ERR_INVALID_ARGUMENT (null out / mats with n_mats > 0,
 * non-positive dims), MFSDP_ERR_UNSUPPORTED (dtype, or a size beyond the
 * 32-bit element indexing of the kernels).
 */
mfsdp_status_t mfsdp_muon_workspace_size(const mfsdp_matrix_t* mats,
                                         int64_t n_mats, mfsdp_dtype_t dtype,
                                         size_t* out_bytes);

/*
 * Owner-local Muon step over `n_mats` whole matrices (host array `mats`).
 *
 * For each matrix, in fp32 arithmetic (arxivlens Abstract: Muon orthogonalizes
 * momentum-smoothed updates with Newton-Schulz on the whole matrix):
 *   M' = beta*M + G                                  (stored to momentum)
 *   U  = G + beta*M'   (nesterov != 0)   or   U = M'
 *   X0 = U / (||U||_F + MFSDP_NS_EPS), transposed to m x n when rows > cols
 *   ns_steps times:  A = X X^T;  B = b*A + c*A*A;  X = a*X + B*X
 *   O  = X (transposed back)
 *   W' = (1 - lr*weight_decay)*W - lr*scale*O        (stored to weight)
 * With dtype BF16, X, A and B are rounded to bf16 (round to nearest even)
 * between the products, which accumulate in fp32.  Matrices are independent:
 * results do not depend on their order in the list or on how the library
 * groups them.
 *
 * workspace        device, >= mfsdp_muon_workspace_size bytes, 256-byte
 *                  aligned; contents are scratch and are overwritten.
 * n_mats == 0      (a rank that owns no matrix) returns MFSDP_OK, no work.
 * Streams: when a list has few rounds of tiles, the Newton-Schulz iterations
 * run as up to four flop-balanced groups of matrices.  The first group runs on
 * `stream`; the others run on auxiliary streams that the library owns, one
 * set per (device, caller stream), created on first use at the default
 * priority and kept until the process ends.  The auxiliary streams are forked
 * from `stream` with an event and joined back into it before the call
 * returns, so all the work is ordered after earlier work on `stream` and
 * before later work on it; calls on different caller streams share no
 * auxiliary stream.  The environment variable MFSDP_NS_GROUPS=1 keeps
 * everything on `stream`.  Calls may come from several host threads (one
 * caller stream per thread at a time); the pool lookup is guarded by a mutex.
 * Launch tables: each call uploads its descriptors and tile tables into the
 * workspace with hipMemcpyAsync from host memory that lives only during the
 * call (the HIP runtime stages such a copy before it returns).  A stream that
 * is being captured into a graph is therefore refused with
 * MFSDP_ERR_UNSUPPORTED, before anything is enqueued.
 * MFSDP_LOG=1 prints each call's launch plan (groups, tiles per launch,
 * padded shapes, workspace bytes) to stderr.
 * Validation: non-null weight/grad/momentum, rows, cols >= 1, 16-byte
 * aligned buffers, pairwise non-overlapping weight/grad/momentum/update_out/
 * workspace across the whole list, ns_steps in [0, 100], finite lr, beta,
 * weight_decay, a, b, c and scale, scale > 0.
 */
mfsdp_status_t mfsdp_muon_step(const mfsdp_matrix_t* mats, int64_t n_mats,
                               mfsdp_dtype_t dtype, float lr, float beta,
                               int nesterov, float weight_decay, int ns_steps,
                               float a, float b, float c, void* workspace,
                               size_t workspace_bytes, hipStream_t stream);

/*
 * The same step for callers that cannot allocate device memory: code that
 * may not call hipMalloc (tight serving loops, harnesses that forbid it, a
 * caller with no free HBM left to hand out a workspace).  It takes the
 * arguments of mfsdp_muon_step except the workspace, and uses instead a
 * static device array of MFSDP_NOALLOC_SCRATCH_BYTES (256 MiB) that the
 * library holds on every GPU it runs on, from the loading of its code object
 * on that GPU until the process ends.
 *   - A list whose workspace (mfsdp_muon_workspace_size) exceeds
 *     MFSDP_NOALLOC_SCRATCH_BYTES is refused with MFSDP_ERR_WORKSPACE before
 *     the device is touched: split the list, or use mfsdp_muon_step.
 *   - The call allocates no device or pinned host memory and creates no
 *     stream or event: every Newton-Schulz group runs on `stream` (results
 *     are bitwise those of mfsdp_muon_step, which does not depend on the
 *     grouping).  The only allocations are the host-side launch tables.
 *   - All calls on one GPU share that GPU's array, which keeps the last
 *     call's contents (nothing in it needs to start at zero: each call writes
 *     what it reads).  Calls that overlap on one GPU -- on two streams, or
 *     from two threads -- race on it and give undefined results; order them
 *     on one stream.
 *   - Like mfsdp_muon_step, a stream under graph capture is refused.
 * Validation and every other error are those of mfsdp_muon_step.
 */
#define MFSDP_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)

mfsdp_status_t mfsdp_muon_step_noalloc(const mfsdp_matrix_t* mats, int64_t n_mats,
                                       mfsdp_dtype_t dtype, float lr, float beta,
                                       int nesterov, float weight_decay, int ns_steps,
                                       float a, float b, float c, hipStream_t stream);

/*
 * Decoupled AdamW on a packed fp32 tail of n elements (arxivlens Abstract:
 * the tensors that are not 2D matrices go to tail owners in packed form and
 * keep the AdamW optimizer).
 * Elementwise, with t = step (>= 1):
 *   p  <- p * (1 - lr*weight_decay)
 *   m  <- beta1*m + (1-beta1)*g
 *   v  <- beta2*v + (1-beta2)*g*g
 *   p  <- p - lr * (m / (1-beta1^t)) / (sqrt(v / (1-beta2^t)) + eps)
 * param, exp_avg, exp_avg_sq are device fp32[n] updated in place, grad is
 * device fp32[n] read only; all 16-byte aligned and non-overlapping.
 * n == 0 (an owner with no tail) returns MFSDP_OK without touching the device.
 * Validation: non-null pointers for n > 0, n >= 0, step >= 1, finite
 * hyperparameters, beta1 and beta2 in [0, 1), eps >= 0; n > 2^40 returns
 * MFSDP_ERR_UNSUPPORTED.
 */
mfsdp_status_t mfsdp_adamw_tail(float* param, const float* grad,
                                float* exp_avg, float* exp_avg_sq, int64_t n,
                                float lr, float beta1, float beta2, float eps,
                                float weight_decay, int64_t step,
                                hipStream_t stream);

/*
 * Balance-aware owner planner (host only; touches no device).
 *
 * Source: arxivlens page, Methodology (a balance-aware owner planner assigns
 * ownership by bytes and by work); gist.science summaries, "Méthodologie",
 * part 2, first mechanism (a global planner chooses owners so that resident
 * bytes and optimizer work are balanced across the ranks).  The pages give no
 * algorithm; this one is greedy longest-processing-time-first scheduling
 * (Graham 1969) under a per-owner byte cap.
 *
 * Items are whole: a 2D matrix or a tail tensor, each going to exactly one of
 * n_ranks owners.
 *   cost_ms[n_items]   host, predicted optimizer-step time of each item on its
 *                      owner (for example measured per shape); finite, >= 0
 *   bytes[n_items]     host, resident bytes of each item on its owner (weight,
 *                      gradient and optimizer state); >= 0
 *   byte_slack         each owner's bytes stay within
 *                      cap = ceil((1 + byte_slack) * max(total/n_ranks, largest))
 *                      when any owner can take the item under it
 * In order of decreasing cost (ties: more bytes first, then lower index), each
 * item goes to the owner with the least predicted time among those it keeps
 * under the cap (ties: lower rank); when none can, to the owner with the
 * fewest bytes.  Without a binding cap the largest predicted time is within
 * (4/3 - 1/(3 n_ranks)) of the optimum.  Deterministic.
 * Outputs (host): owner[n_items] in [0, n_ranks); rank_ms[n_ranks] = summed
 * cost per owner; rank_bytes[n_ranks] = summed bytes per owner.
 * Errors: MFSDP_ERR_INVALID_ARGUMENT (n_items < 0, n_ranks < 1, null
 * pointers, negative or non-finite cost, negative bytes or slack).
 */
mfsdp_status_t mfsdp_plan_owners(const double* cost_ms, const int64_t* bytes,
                                 int64_t n_items, int32_t n_ranks,
                                 double byte_slack, int32_t* owner,
                                 double* rank_ms, int64_t* rank_bytes);

/*
 * Packed tail layout (host only).  Source: arxivlens Abstract and gist.science
 * "Méthodologie", part 1: vectors and other non-2D tensors go, grouped, to a
 * tail owner, which runs AdamW on the packed buffer.
 * Tensor i of numel[i] fp32 elements occupies elements
 * [offsets[i], offsets[i] + numel[i]) of the packed buffer; segments follow
 * in order, each starting on a 16-byte (4-element) boundary.  *total is the
 * packed length (the last segment rounded up to 4).
 * Errors: MFSDP_ERR_INVALID_ARGUMENT (n < 0, null pointers, numel < 0).
 */
mfsdp_status_t mfsdp_tail_layout(const int64_t* numel, int64_t n,
                                 int64_t* offsets, int64_t* total);

/*
 * Gather tensors into a packed fp32 tail (device copy on `stream`).
 *   src[n]      host array of device pointers, tensor i of numel[i] fp32
 *               elements (4-byte aligned; may be NULL when numel[i] == 0)
 *   offsets[n]  host, element offsets in the packed buffer: multiples of 4,
 *               segments [offset, offset + round_up(numel, 4)) in bounds and
 *               pairwise disjoint (mfsdp_tail_layout gives such offsets)
 *   packed      device, packed_numel fp32 elements, 16-byte aligned; must not
 *               overlap any source
 * Each segment receives its tensor followed by zeros up to the next 4-element
 * boundary; elements outside every segment are left unchanged.
 * Errors: MFSDP_ERR_INVALID_ARGUMENT, MFSDP_ERR_ALIAS (overlapping segments,
 * or a source overlapping the packed buffer), MFSDP_ERR_HIP.
 */
mfsdp_status_t mfsdp_tail_pack(const float* const* src, const int64_t* numel,
                               const int64_t* offsets, int64_t n, float* packed,
                               int64_t packed_numel, hipStream_t stream);

/*
 * Scatter a packed fp32 tail back into its tensors (device copy on `stream`):
 * dst[i][0 .. numel[i]) = packed[offsets[i] ..].  Same argument rules as
 * mfsdp_tail_pack; the destinations must not overlap each other or the
 * packed buffer (MFSDP_ERR_ALIAS).
 */
mfsdp_status_t mfsdp_tail_unpack(const float* packed, int64_t packed_numel,
                                 float* const* dst, const int64_t* numel,
                                 const int64_t* offsets, int64_t n,
                                 hipStream_t stream);

/*
 * Preconditioner statistics of Shampoo-type matrix optimizers on the owner.
 *
 * Source: gist.science summaries (French and Portuguese pages),
 * "Problématique" (Shampoo and SOAP, like Muon, take the whole 2D gradient
 * as input) and "Contributions clés", item "Généralité" (the owner-shaped
 * layout is not tied to one optimizer).  The arxivlens page names only Muon.  The pages give no formulas; the
 * statistics are the textbook Shampoo ones (Gupta, Koren and Singer 2018),
 * with SOAP's exponential moving average as the beta/alpha form.
 *
 * One whole gradient of the list, row-major rows x cols in the call's dtype:
 *   grad    device, read only
 *   left    device fp32 rows x rows, updated in place:  L <- beta*L + alpha*G G^T
 *   right   device fp32 cols x cols or NULL, updated:   R <- beta*R + alpha*G^T G
 * The products accumulate in fp32 from the stored gradient values (bf16 or
 * fp32); L and R stay exactly symmetric (the upper triangle is computed and
 * mirrored).  beta == 0 overwrites L and R without reading them.
 */
typedef struct mfsdp_stats_matrix {
  const void* grad;
  float* left;
  float* right;
  int64_t rows;
  int64_t cols;
} mfsdp_stats_matrix_t;

/* Workspace bytes for mfsdp_shampoo_stats (host only): two zero-padded copies
 * of each gradient (G and its transpose, 256-padded) and launch tables.
 * n_mats == 0 gives 0.  Errors: MFSDP_ERR_INVALID_ARGUMENT, MFSDP_ERR_UNSUPPORTED
 * (dtype, or a size beyond the 32-bit offsets of the kernels). */
mfsdp_status_t mfsdp_stats_workspace_size(const mfsdp_stats_matrix_t* mats,
                                          int64_t n_mats, mfsdp_dtype_t dtype,
                                          size_t* out_bytes);

/* Statistics update over the list, enqueued on `stream`.  workspace: device,
 * >= mfsdp_stats_workspace_size bytes, 256-byte aligned, scratch.  Like
 * mfsdp_muon_step, the call uploads its launch tables from host memory and
 * refuses a stream under graph capture (MFSDP_ERR_UNSUPPORTED).
 * Validation before any launch: rows, cols >= 1; non-null grad and left;
 * naturally aligned buffers; grad/left/right/workspace pairwise disjoint
 * across the list (MFSDP_ERR_ALIAS); finite beta and alpha. */
mfsdp_status_t mfsdp_shampoo_stats(const mfsdp_stats_matrix_t* mats, int64_t n_mats,
                                   mfsdp_dtype_t dtype, float beta, float alpha,
                                   void* workspace, size_t workspace_bytes,
                                   hipStream_t stream);

/* Static, human-readable name of a status code. */
const char* mfsdp_status_string(mfsdp_status_t status);

/* Thread-local detail of the last failure on this thread ("" if none). */
const char* mfsdp_last_error(void);

/*
 * Kernel timing for measurement tools.  Kernels of the library fall into the
 * kinds below.  While timing is enabled on a thread, every launch that thread
 * makes is bracketed by a pair of hipEvents recorded on the launch stream;
 * mfsdp_timing_read synchronizes those events and returns, per kind, the
 * summed milliseconds and the number of launches since the last reset.
 * Events are created lazily by the library (no device-memory allocation) and
 * kept per thread.  Not needed for normal use.
 */
typedef enum mfsdp_kernel_kind {
  MFSDP_KERNEL_MOMENTUM = 0,  /* momentum + Nesterov + norm partials */
  MFSDP_KERNEL_NORM = 1,      /* per-matrix norm finalization        */
  MFSDP_KERNEL_GRAM = 2,      /* A = X X^T                           */
  MFSDP_KERNEL_POLY = 3,      /* B = b A + c A A                     */
  MFSDP_KERNEL_UPDATE = 4,    /* X = a X + B X, all but the last     */
  MFSDP_KERNEL_APPLY = 5,     /* apply when ns_steps == 0            */
  MFSDP_KERNEL_ADAMW = 6,     /* AdamW tail                          */
  MFSDP_KERNEL_FINAL = 7,     /* last update, applies W (2 launches) */
  MFSDP_KERNEL_STATS_PREP = 8,/* gradient copies for the statistics   */
  MFSDP_KERNEL_SYRK = 9,      /* L, R statistics products            */
  MFSDP_KERNEL_SMALL = 10,    /* whole NS chain + apply of small matrices */
  MFSDP_KERNEL_KINDS = 11
} mfsdp_kernel_kind_t;

mfsdp_status_t mfsdp_timing_enable(int enable);
mfsdp_status_t mfsdp_timing_reset(void);
mfsdp_status_t mfsdp_timing_read(mfsdp_kernel_kind_t kind, double* total_ms,
                                 int64_t* launches);

/*
 * Measurement only: the sustained bf16 MFMA rate of this GPU with no memory
 * traffic, the practical ceiling for the Newton-Schulz products (under
 * sustained MFMA load the clock settles below the one at which the dense peak
 * is quoted).  Launches `blocks` workgroups of 8 waves on `stream`; each wave
 * issues 8 * iters v_mfma_f32_32x32x16_bf16 (32768 flops each) on register
 * operands and writes one float to out[8 * block + wave] (device, blocks * 8
 * floats, 4-byte aligned).  The caller times the launch (for example with
 * hipEvents on `stream`).  Errors: MFSDP_ERR_INVALID_ARGUMENT (NULL or
 * misaligned out, blocks outside [1, 65536], iters outside [1, 2^20], or
 * blocks * iters above 2^28, which bounds a launch to about half a second),
 * MFSDP_ERR_HIP.
 */
mfsdp_status_t mfsdp_mfma_probe(float* out, int64_t blocks, int iters,
                                hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MFSDP_H_ */
