/*
 * lowbit.h -- C ABI of the packed low-bit GEMV/GEMM library for MI355X (gfx950).
 *
 * The library multiplies fp16/bf16 activations by weights kept in packed
 * group-scaled low-bit form and never expands them to a dense matrix in
 * memory: the sign bits / trits are decoded inside the matrix kernels and
 * multiplied by their group's FP16 scale there.
 *
 * Formats (value maps fixed by the pages this library follows):
 *  - LOWBIT_Q1_G128, "Binary g128": one sign bit per weight, stored bit 0 means
 *    -scale and bit 1 means +scale; one FP16 scale per 128 weights, so
 *    1 + 16/128 = 1.125 bits per weight (lnrk.cn page, Binary g128 section;
 *    aberweb.com page, section 4.1 and Table 2).
 *  - LOWBIT_TQ2_G128, "Ternary g128 in 2-bit slots": t in {-1,0,+1} stored as
 *    the 2-bit code c = t + 1 (code 3 unused), one FP16 scale per 128 weights,
 *    2.125 bits per weight (ksqn.cn page, ternary weight representation and
 *    "current limitations").
 *  - LOWBIT_TQ5_G128, "Ternary g128, 5 trits per byte": base-3 digits
 *    d = t + 1, five per byte (3^5 = 243 <= 256, cnblogs.com page, section
 *    2.4), ceil(K/5) bytes per row, one FP16 scale per 128 weights.
 *  A group is 128 consecutive weights along K inside one row, so K must be a
 *  multiple of 128.
 *
 * Blob ("packed weights"): headerless, exactly packed_bytes_lowbit(fmt,N,K)
 * bytes: plane A (signs / codes / trit bytes in the device layout v2, an
 * arrangement of the bits chosen for 128-bit coalesced loads and cheap
 * in-register decode) followed by plane B, the N*K/128 FP16 scale bit
 * patterns in the order of the kernels' units (16 rows x 4 groups, or 5 for
 * tq5, contiguous).  pack_* writes it, unpack_lowbit inverts it exactly.
 *
 * Product: for m < M, n < N
 *     Y[m][n] = sum_k X[m][k] * t[n][k] * s[n][k/128]
 * (aberweb.com page, section 4.1: the stored bits become signed values
 * multiplied by the FP16 scale of their 128-weight group; ksqn.cn page:
 * ternary weights are {-1, 0, +1} times the group scale).  W row n is
 * output feature n (nn.Linear order); X is M x K and Y is M x N, both
 * row-major and contiguous.  Y is overwritten.  Accumulation is fp32
 * with every product exact (weights are decoded to exact +-1 / 0 and the
 * FP16 scale is applied in fp32 once per group); an fp16 Y is rounded to
 * nearest even from the fp32 result.  Results are deterministic for a given
 * input, shape and device.
 *
 * Errors: every call validates its arguments before doing anything and
 * returns LOWBIT_OK (0) or a negative status; on error nothing is written and
 * nothing is launched.  No C++ exception, abort or exit crosses this ABI.
 * Thread safety: all calls are reentrant; the library keeps no state besides
 * a lazily filled, lock-protected cache of device properties.
 */
#ifndef LOWBIT_H
#define LOWBIT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LOWBIT_ABI_VERSION 7

typedef enum { LOWBIT_Q1_G128 = 1, LOWBIT_TQ2_G128 = 2, LOWBIT_TQ5_G128 = 3 } lowbit_format;
typedef enum { LOWBIT_F16 = 1, LOWBIT_BF16 = 2, LOWBIT_F32 = 3 } lowbit_dtype;

enum {
  LOWBIT_OK = 0,
  LOWBIT_ERR_NULL = -1,   /* a required pointer is NULL                               */
  LOWBIT_ERR_ENUM = -2,   /* unknown format or dtype value                            */
  LOWBIT_ERR_SHAPE = -3,  /* negative M/N/K, or K not a multiple of 128               */
  LOWBIT_ERR_VALUE = -4,  /* code outside the format's set (pack), tq2 code 3, tq5 byte
                             >= 243 or non-zero tq5 padding trit (unpack)             */
  LOWBIT_ERR_SIZE = -5,   /* a buffer is smaller than required                        */
  LOWBIT_ERR_ALIGN = -6,  /* W or X not 16-byte aligned, Y not aligned to its dtype     */
  LOWBIT_ERR_DTYPE = -7,  /* unsupported x / y dtype combination                       */
  LOWBIT_ERR_DEVICE = -8  /* the HIP runtime reported an error                         */
};

/* Library ABI version (LOWBIT_ABI_VERSION of the build).  The formats it
 * serves are those of the lnrk.cn page (Binary g128 section), the ksqn.cn
 * page (ternary g128) and the cnblogs.com page (section 2.4, 5 trits per
 * byte). */
int lowbit_abi_version(void);

/* Static string describing a status code; never NULL.  The value checks it
 * names follow the value maps of the lnrk.cn page (Binary g128 section) and
 * the ksqn.cn page ("current limitations": ternary codes in 2-bit slots). */
const char *lowbit_strerror(int status);

/* Size in bytes of a packed blob: plane A + N*(K/128)*2.
 *   q1: N*K/8 + N*(K/128)*2      (1.125 bits per weight: one sign bit per
 *       weight and one FP16 scale per 128, lnrk.cn page, Binary g128 section
 *       and its memory table; the aberweb.com page, Table 2, gives the same
 *       18/128 bytes per weight for the 8B model)
 *   tq2: N*K/4 + N*(K/128)*2     (2.125 bits per weight: ternary in 2-bit
 *       slots, ksqn.cn page, "current limitations")
 *   tq5: N*ceil(K/5) + N*(K/128)*2  (5 trits per byte, cnblogs.com page,
 *       section 2.4)
 * Returns a negative status on a bad format or shape. */
int64_t packed_bytes_lowbit(int fmt, int64_t N, int64_t K);

/* Pack codes and scales (host memory in, host memory out): the value maps
 * of the lnrk.cn page (Binary g128 section: bit 1 -> +scale, bit 0 ->
 * -scale), the ksqn.cn page (ternary {-1,0,+1} with a g128 FP16 scale, 2-bit
 * slots) and the cnblogs.com page (section 2.4: 5 trits per byte).
 *   codes:  int8 [N][K], row-major; q1: values in {-1,+1}; tq2/tq5: {-1,0,+1}
 *   scales: uint16 [N][K/128], FP16 bit patterns, stored bit-exactly
 *   out:    caller-owned, at least packed_bytes_lowbit(fmt, N, K) bytes
 * Returns LOWBIT_ERR_VALUE (and writes nothing) if any code is out of set.
 * Uses up to hardware_concurrency() host threads.                         */
int pack_q1_g128(const int8_t *codes, const uint16_t *scales, int64_t N, int64_t K,
                 void *out, int64_t out_bytes);
int pack_tq2_g128(const int8_t *codes, const uint16_t *scales, int64_t N, int64_t K,
                  void *out, int64_t out_bytes);
int pack_tq5_g128(const int8_t *codes, const uint16_t *scales, int64_t N, int64_t K,
                  void *out, int64_t out_bytes);

/* Import of MLX's grouped affine 1-bit format (1.25 bits/weight): per group
 * of 128 weights along K a scale a and a bias b, weight = a * q + b with
 * q in {0, 1} (lnrk.cn page, MLX packing paragraph; aberweb.com page,
 * summary section 2).
 *   wq: host, uint32 [N][K/32]; bit k % 32 of word k / 32 holds q[n][k]
 *   scales, biases: host, [N][K/128] in sb_dtype (LOWBIT_F16, LOWBIT_BF16 or
 *     LOWBIT_F32 bit patterns)
 *   out: host, packed_bytes_lowbit(LOWBIT_Q1_G128, N, K) bytes: the Binary
 *     g128 blob of the same matrix (bit q -> code 2q - 1, scale s = -b).
 * A group converts exactly when a = -2 b (its two values are -s and +s)
 * and -b is an FP16 value; any other group returns LOWBIT_ERR_VALUE and
 * nothing is written.  Other errors as for pack_*. */
int import_mlx_q1_g128(const uint32_t *wq, const void *scales, const void *biases, int sb_dtype,
                       int64_t N, int64_t K, void *out, int64_t out_bytes);

/* Exact inverse of pack_* (host memory): the same value maps read back
 * (lnrk.cn page, Binary g128 section; ksqn.cn page, "current limitations";
 * cnblogs.com page, section 2.4, whose byte of 5 trits has 243 valid values).
 * codes_out int8 [N][K] and scales_out uint16 [N][K/128] are caller-owned;
 * either may be NULL to skip it. */
int unpack_lowbit(int fmt, const void *packed, int64_t packed_bytes, int64_t N, int64_t K,
                  int8_t *codes_out, uint16_t *scales_out);

/* Workspace that lets gemv_lowbit take its fastest path for this problem
 * (0 = the fastest path needs none).  Decode is bound by streaming the
 * weights (aberweb.com page, sections 2 and 4.4), so small matrices cut K
 * across workgroups to keep every compute unit streaming.  The decode product may cut K into
 * ranges handled by different workgroups; their fp32 partial sums live here,
 * after 32 KiB of arrival counters at its start.  The size does not depend
 * on the device or on the activation dtype; base-3 (tq5) weights never use
 * it.
 * Returns a negative status on a bad format or shape. */
int64_t gemv_workspace_bytes_lowbit(int fmt, int64_t M, int64_t N, int64_t K);

/* Decode GEMV: Y = X W^T for small batches (tuned for M <= 16; any M works;
 * more than 16 tokens run as consecutive 16-token launches).  The packed
 * bits are decoded inside the matrix kernel and multiplied by their group's
 * FP16 scale there, with no dense weight tensor (aberweb.com page, section
 * 4.1); token generation is bandwidth-bound (aberweb.com page, section 2).
 *   Wp: device, packed blob of this (fmt, N, K), 16-byte aligned
 *   X:  device, M x K, x_dtype LOWBIT_F16 or LOWBIT_BF16, 16-byte aligned
 *   Y:  device, M x N, y_dtype LOWBIT_F32 or LOWBIT_F16
 *   workspace: caller-owned device memory, 16-byte aligned, or NULL.  It
 *   must be zero-filled before its first use (it holds arrival counters that
 *   every call leaves at zero again); calls that may run concurrently need
 *   separate workspaces.  With at least gemv_workspace_bytes_lowbit() bytes
 *   the call may split K across workgroups; with less, or NULL, it takes a
 *   path that needs none.  Results obey the same bound and are deterministic
 *   for a given workspace size either way.
 *   hip_stream: hipStream_t to launch on (NULL = default stream); the call is
 *   asynchronous with respect to the host.
 * M*N == 0 returns LOWBIT_OK without launching; K == 0 writes Y = 0.       */
int gemv_lowbit(int fmt, const void *Wp, const void *X, int x_dtype, void *Y, int y_dtype,
                int64_t M, int64_t N, int64_t K, void *workspace, int64_t workspace_bytes,
                void *hip_stream);

/* Decode GEMV for callers that cannot allocate: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  It is
 * gemv_lowbit with its workspace in a device array inside the library
 * (8 MiB + 32 KiB on each device it runs on, held until the process ends)
 * instead of a caller's buffer: same arguments without the workspace, same
 * kernels, plans and results as gemv_lowbit given a workspace of that size.
 * It calls no hipMalloc, hipFree or allocating library routine.  A problem
 * whose fastest path would need a larger workspace is refused with
 * LOWBIT_ERR_SIZE (no shape needs one today).  All calls on one device share
 * that device's array and leave its counters at zero: calls that may overlap
 * in time on one device (two streams, two host threads) race on it. */
int gemv_lowbit_noalloc(int fmt, const void *Wp, const void *X, int x_dtype, void *Y, int y_dtype,
                        int64_t M, int64_t N, int64_t K, void *hip_stream);

/* Matrices one fused decode call may cover (the query / key / value or
 * gate / up projections of a block share x; lnrk.cn page, DSpark section). */
#define LOWBIT_MAX_FUSED 4

/* Workspace for gemv_multi_lowbit over these matrices (same meaning and
 * rules as gemv_workspace_bytes_lowbit; decode is bandwidth-bound,
 * aberweb.com page, section 2).  Ns: host array of count row counts.
 * Returns a negative status on a bad format, count or shape. */
int64_t gemv_multi_workspace_bytes_lowbit(int fmt, int count, const int64_t *Ns, int64_t M, int64_t K);

/* Fused decode GEMV: Y_i = X W_i^T for i < count (1..LOWBIT_MAX_FUSED), for
 * matrices that share the activations X and K, such as the query, key and
 * value projections, or the gate and up projections, of a transformer block
 * (serving with draft-token verification makes M small but above one:
 * lnrk.cn page, DSpark section; ksqn.cn page).  One launch covers the row
 * tiles of all of them, so the fixed cost of a launch is paid once.
 *   Ws: host array of count device pointers, the packed blob of (fmt, Ns[i], K)
 *   Ns: host array of count row counts (0 allowed: that matrix is skipped)
 *   Ys: host array of count device pointers, M x Ns[i] each, y_dtype
 *   X, x_dtype, y_dtype, M, K, workspace, hip_stream: as for gemv_lowbit
 * Each Y_i obeys the same bound as gemv_lowbit.  Errors as for gemv_lowbit,
 * checked for every matrix before anything is launched; a count outside
 * 1..LOWBIT_MAX_FUSED is LOWBIT_ERR_SHAPE. */
int gemv_multi_lowbit(int fmt, int count, const void *const *Ws, const int64_t *Ns, const void *X,
                      int x_dtype, void *const *Ys, int y_dtype, int64_t M, int64_t K,
                      void *workspace, int64_t workspace_bytes, void *hip_stream);

/* Workspace that lets gemm_lowbit balance its work over the whole chip
 * (prompt processing is compute-bound, aberweb.com page, summary section 3,
 * so every compute unit should multiply until the end): the
 * (tile, 128-weight group) work items are cut into one contiguous range per
 * workgroup slot, and tiles split between two ranges are summed through this
 * memory (64 KiB of arrival counters, then two fp32 output tiles per slot:
 * 128 x 256 for q1 and tq2, 128 x 128 for tq5).  For q1 it also holds bf16 x
 * converted once per call into two fp8 pieces per value with one power-of-two
 * scale per 32 values (2 bytes + 1/32 byte per value of x padded to 128-row
 * tiles), which the q1 kernel multiplies against fp4 +-1 weights: that is
 * exact for every value within 2^7 of its 32-value block's largest, and
 * keeps the error below 2^-12 of the bound's sum otherwise.  Depends on the
 * format, on M and K for q1, and on the device's compute-unit count (256
 * assumed when no device is visible).  Returns a negative status on a bad
 * format or shape. */
int64_t gemm_workspace_bytes_lowbit(int fmt, int64_t M, int64_t N, int64_t K);

/* Prefill GEMM: Y = X W^T for large batches (M = prompt tokens), a dense
 * contraction on the matrix cores: prompt processing is compute-bound
 * (aberweb.com page, summary section 3) and the bits are decoded inside the
 * matrix kernel (aberweb.com page, section 4.1).  Same
 * arguments and rules as gemv_lowbit, including the workspace: caller-owned,
 * 16-byte aligned, zero-filled before its first use (every call leaves its
 * counters zero again), one per concurrently running call.  With at least
 * gemm_workspace_bytes_lowbit() bytes the work is balanced across the chip
 * (and q1 with bf16 x takes the fp8-piece path); with less, or NULL, each
 * workgroup takes whole tiles with exact bf16 operands.  Results are
 * deterministic for a given workspace size either way. */
int gemm_lowbit(int fmt, const void *Wp, const void *X, int x_dtype, void *Y, int y_dtype,
                int64_t M, int64_t N, int64_t K, void *workspace, int64_t workspace_bytes,
                void *hip_stream);

/* ---- Plans: which kernel a product call would launch, and how it splits the
 * work.  Decode (small M) streams the weights and is bandwidth-bound, prefill
 * (large M) is compute-bound (aberweb.com page, sections 2 and 4.4 and
 * summary section 3), so the two products take different kernels and work
 * splits; these calls report them without launching anything. */
typedef enum {
  LOWBIT_KERNEL_NONE = 0,         /* nothing to launch (M * N == 0)                        */
  LOWBIT_KERNEL_GEMV_STAGED = 1,  /* decode, x staged in LDS once per workgroup            */
  LOWBIT_KERNEL_GEMV_SPLIT = 2,   /* decode, row blocks x K ranges, x staged per block     */
  LOWBIT_KERNEL_GEMV_WIDE = 3,    /* decode, x read straight into registers (9..16 tokens) */
  LOWBIT_KERNEL_GEMV_TQ5 = 4,     /* decode, base-3 weights                                */
  LOWBIT_KERNEL_GEMV_TQ5_ONE = 5, /* decode, base-3 weights, one token, x in LDS           */
  LOWBIT_KERNEL_GEMM = 6,         /* prefill                                               */
  LOWBIT_KERNEL_FILL_ZERO = 7,    /* K == 0: Y = 0                                         */
  LOWBIT_KERNEL_GEMV_KSLICE = 8   /* decode, 9..16 tokens, each wave one chunk of K of all  *
                                   * the workgroup's row tiles, x in registers              */
} lowbit_kernel;

typedef enum {
  LOWBIT_OPERANDS_NONE = 0,
  LOWBIT_OPERANDS_F16 = 1,     /* exact f16 operands on v_mfma_f32_16x16x32_f16            */
  LOWBIT_OPERANDS_BF16 = 2,    /* exact bf16 operands on v_mfma_f32_16x16x32_bf16          */
  LOWBIT_OPERANDS_FP8_FP4 = 3,   /* bf16 x as two fp8 pieces, weights as fp4, scaled 16x16x128 */
  LOWBIT_OPERANDS_FP8X3_FP4 = 4  /* fp16 x as three fp8 pieces, weights as fp4, the same MFMA    */
} lowbit_operands;

typedef struct {
  int kernel;            /* lowbit_kernel of the call's main launch                     */
  int launches;          /* kernel launches the call issues in all                      */
  int grid;              /* workgroups of the main launch (of its first 16-token block) */
  int threads;           /* work-items per workgroup                                    */
  int lds_bytes;         /* dynamic LDS bytes per workgroup                             */
  int token_slots;       /* token rows one launch covers (1, 2, 4, 8 or 16; GEMM 128)   */
  int operands;          /* lowbit_operands                                             */
  int whole_tiles;       /* 1: addresses for whole 16-row tiles and whole 4-group chunks */
  int tiles_per_wave;    /* row tiles (16 rows each) a wave holds per unit of work      */
  int waves;             /* waves per workgroup                                         */
  int waves_per_tile;    /* waves of one workgroup that split one tile set's K          */
  int k_ranges;          /* K ranges cut across workgroups (partial sums in workspace)  */
  int groups_per_range;  /* 128-weight groups per K range, or per wave of a wave-row    */
  int groups_per_pass;   /* groups of x staged in LDS per pass (0: not staged)          */
  int ring;              /* units of packed weights in flight per wave                  */
  int items_per_wg;      /* GEMM: (tile, group) items per workgroup (G: whole tiles)    */
  int x_pieces;          /* GEMM: 1 when x is converted to fp8 pieces first             */
  int lds_offsets[3];    /* staged decode kernel: scale/correction, x and reduction areas */
  int reserved[4];
} lowbit_plan;

/* The plan gemv_multi_lowbit (count matrices; count 1 is gemv_lowbit) would
 * follow (decode, bandwidth-bound: aberweb.com page, section 2) with a workspace of workspace_bytes bytes on the current device
 * (256 compute units and one workgroup per CU when no device is visible).
 * Ns: host array of count row counts.  Nothing is launched or allocated.
 * Returns the status the product call would return for these shapes and
 * dtypes (pointer checks aside); out is filled on LOWBIT_OK. */
int lowbit_gemv_plan(int fmt, int count, const int64_t *Ns, int x_dtype, int y_dtype, int64_t M, int64_t K,
                     int64_t workspace_bytes, lowbit_plan *out);

/* The same for gemm_lowbit (prefill, compute-bound: aberweb.com page, summary
 * section 3). */
int lowbit_gemm_plan(int fmt, int x_dtype, int y_dtype, int64_t M, int64_t N, int64_t K, int64_t workspace_bytes,
                     lowbit_plan *out);

#ifdef __cplusplus
}
#endif
#endif /* LOWBIT_H */
