/*
 * qgemv.h — C ABI of the MI355X (gfx950) MLX-affine quantized row product.
 *
 * The operation (one handle = one quantized matrix, or a stack of experts):
 *
 *   q[n,k]  = code k of row n: bits [k*bits, k*bits+bits) of the row's
 *             bitstream, low code first, the bitstream cut into little-endian
 *             32-bit words; a row of K codes ends on a word.
 *   w[n,k]  = scale[n, k/group] * q[n,k] + bias[n, k/group]
 *   y[i,n]  = epi( sum_k w[n,k] * x[i,k] )   for the rows i of a 1..16-row
 *             activation window, in fp32 with fp32 group sums.
 *
 * Sources, on "Qwen3.8-Flash-Next faster kernels in Zig engine - #788":
 *  - commit "...row kernel at every MLX width": every MLX affine width
 *    (2, 3, 4, 5, 6, 8 bits) at groups of 32, 64 and 128; 3- and 5-bit rows
 *    hold eight codes in three or five bytes, low code first; a row ends on a
 *    word; a strided call writes one member of a fused stack straight into
 *    the stack output; options relu2 and indexed slots; a row's bits are the
 *    same alone and inside 2-, 3-, 8- and 16-row windows.
 *  - commit "...lane kernel formats" (Layout.y_stride): a row stride below N
 *    is refused; a strided write leaves the gaps untouched.
 * and on "Qwen3.8-Flash-Next support for oQ in Zig engine - #774":
 *  - "What this changes", item 3: every width kernel is resolved when the
 *    weights are admitted ("fail closed"), so a bad width refuses the
 *    handle, never a request; refusals are named.
 *  - "Exactness", item "Precision": activations stay bf16, group sums fp32.
 *
 * Memory and ownership.  Every array argument is a DEVICE pointer (HIP
 * device memory, e.g. a torch tensor's data_ptr()).  The library never
 * allocates or frees device memory and never synchronises (the test-only
 * qgemv_check_indices excepted): a handle BORROWS the
 * weight pointers given at create, which must stay valid until
 * qgemv_destroy.  A handle is immutable after create, so runs on different
 * streams may share it.
 *
 * Error behaviour.  Every argument that can be checked on the host is
 * checked before any HIP call; on a refusal nothing is launched and no
 * output is touched.  Run calls enqueue on the given stream and return
 * without waiting; a device-side fault surfaces at the caller's next
 * synchronisation, as usual in HIP.  Statuses are the QGEMV_E_* values;
 * qgemv_strerror names them.
 */
#ifndef QGEMV_H
#define QGEMV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---------------------------------------------------- */
#define QGEMV_OK 0
#define QGEMV_E_ARG (-1)      /* null pointer or handle, bad enum, misuse   */
#define QGEMV_E_BITS (-2)     /* bits not in {2,3,4,5,6,8}                  */
#define QGEMV_E_GROUP (-3)    /* group not in {32,64,128}                   */
#define QGEMV_E_SHAPE (-4)    /* n < 1, k < 1, group does not divide k,
                                 k*bits not a multiple of 32, too large     */
#define QGEMV_E_STRIDE (-5)   /* output row stride below n                  */
#define QGEMV_E_ALIGN (-6)    /* pointer not aligned to its element type    */
#define QGEMV_E_WINDOW (-7)   /* window rows outside 0..16 (0..65 for plain
                                 and strided calls, matrix-core forms)      */
#define QGEMV_E_ALIAS (-8)    /* output overlaps an input                   */
#define QGEMV_E_NOKERNEL (-9) /* no compiled kernel for this shape          */
#define QGEMV_E_HIP (-10)     /* a HIP runtime call failed                  */
#define QGEMV_E_INDEX (-11)   /* an expert index outside [0, n_experts)
                                 (qgemv_check_indices only)                 */

/* ---- epilogues ------------------------------------------------------- */
#define QGEMV_EPI_NONE 0
#define QGEMV_EPI_RELU2 1     /* y > 0 ? y*y : (y is NaN ? y : +0), on fp32 y */

#define QGEMV_MAX_WINDOW 16
#define QGEMV_MAX_PROMPT 65   /* prompt windows: plain and strided calls, matrix-core forms */

/* Weights of one handle.
 *   bits       code width: 2, 3, 4, 5, 6 or 8.
 *   group      codes per scale/bias along K: 32, 64 or 128.
 *   n, k       output columns and reduction length; group | k,
 *              k*bits % 32 == 0, n*k < 2^40.
 *   n_experts  >= 1.  Expert e's arrays follow expert e-1's without gaps.
 *   w          uint32 [n_experts][n][k*bits/32], 16-byte aligned.
 *   scales     bf16 bits [n_experts][n][k/group], 2-byte aligned.
 *   biases     bf16 bits [n_experts][n][k/group], 2-byte aligned.          */
typedef struct qgemv_desc {
  int32_t bits;
  int32_t group;
  int64_t n;
  int64_t k;
  int32_t n_experts;
  const uint32_t* w;
  const uint16_t* scales;
  const uint16_t* biases;
} qgemv_desc;

typedef struct qgemv_handle* qgemv_t;

/* Validate the weights' shape and pointers, resolve the compiled kernel for
 * (bits, group) and fix the launch geometry from (bits, group, n, k) only —
 * never from the window — so a row's bits cannot depend on the window it
 * runs in.  Makes no HIP call (the current device's compute-unit count is
 * read at the first run on each device).
 * Returns QGEMV_OK and *out, or a refusal (then *out is untouched). */
int qgemv_create(const qgemv_desc* d, qgemv_t* out);

/* ---- arithmetic of a handle --------------------------------------------
 * Every form computes, per output, the sum over the row's 32-code units u of
 *   scale(u) * A(u) + bias(u) * X(u),
 * A(u) the fp32 dot of the unit's exact bf16 codes with its activations and
 * X(u) the fp32 sum of its activations ("Exactness", item "Precision", on
 * "...support for oQ..." #774: bf16 activations, fp32 group sums).  The dot
 * form and the matrix-core forms differ in how A(u) is summed and in the
 * order of the folds (the matrix-core forms add each 128-code round's four
 * bias terms first, as one fp32 matrix-core product), so their bits differ;
 * each stays within the fp64 bound.  The two matrix-core forms give the same
 * bits: the matrix cores sum a 16x16x32 product's K as four 8-wide steps in
 * order, which is what the MFMA form's four chained products over a unit do
 * (measured on MI355X, also with activations whose unit dots round, and
 * checked by the GPU tests).  The arithmetic is fixed at create for every
 * window, strided and indexed call of the handle, which is what keeps a
 * row's bits the same alone and inside any window.
 *   QGEMV_ARITH_DOT   lanes own slices of a row's K; v_dot2 chains, then one
 *                     fixed butterfly over the lanes of the row.
 *   QGEMV_ARITH_MFMA  matrix cores: 16x16x32 bf16 products with one window
 *                     row per 4 operand rows; each lane folds its own four
 *                     units in order, no butterfly.  A matrix of few
 *                     columns (n under 32768) splits k
 *                     into 2 or 4 consecutive parts, fixed at create from
 *                     its shape: each part folds from zero and the parts are
 *                     added in order.  Needs k a multiple of
 *                     qgemv_mfma_codes(bits, group) and aligned scales
 *                     and biases (QGEMV_E_NOKERNEL otherwise).
 *   QGEMV_ARITH_WIDE  matrix cores for wide windows: the same loads, K
 *                     split and shape rules as QGEMV_ARITH_MFMA, but after
 *                     the unpack the four lanes of a column trade quarters
 *                     of their units, so each unit is one 16x16x32 product
 *                     over all window rows at once (4 products per 128-code
 *                     round, against 4 per 4 window rows in the MFMA form).
 *                     Each lane folds the units of its column for window
 *                     rows 4q..4q+3.  The trade costs 16 lane swaps per
 *                     round: on MI355X it is faster at 9-16-row windows and
 *                     prompt passes, slower at 1-8 rows.
 *   QGEMV_ARITH_AUTO  the library's choice (what qgemv_create uses): the
 *                     matrix-core arithmetic when the shape and alignment
 *                     allow it, run by the MFMA form's kernels for windows
 *                     of up to 8 rows and by the WIDE form's above (plain,
 *                     strided and gate/up calls; the same bits either way);
 *                     qgemv_arith reports QGEMV_ARITH_MFMA.  Else the dot
 *                     form.                                               */
#define QGEMV_ARITH_AUTO 0
#define QGEMV_ARITH_DOT 1
#define QGEMV_ARITH_MFMA 2
#define QGEMV_ARITH_WIDE 3

/* As qgemv_create, with the arithmetic chosen by the caller. */
int qgemv_create_arith(const qgemv_desc* d, int32_t arith, qgemv_t* out);

/* The arithmetic a handle was created with (QGEMV_ARITH_DOT, _MFMA or
 * _WIDE), or QGEMV_E_ARG for a NULL handle. */
int qgemv_arith(qgemv_t h);

/* The multiple of k that the MFMA form needs, its load group of 128-code
 * rounds (a whole number of 128-byte lines of a row): 512 codes for 2 and 6
 * bits, 1024 for 3 and 5, 256 for 4, 128 for 8 (256 at group 128); 0 for a
 * bad bits or group.  The MFMA form also needs scales and biases 16-byte
 * aligned where a row's scales of one load group fill whole 16-byte pieces,
 * else 4-byte aligned.
 * Speed only (the bits do not change): on matrices of about 100,000 columns
 * or more, 2-, 4- and 8-bit codes run their fastest kernels when k is a
 * multiple of twice this and, at 8/32, 8/64, 4/64, 4/128 and 2/128, the
 * scale and bias arrays are 16-byte (8/32, 4/64, 2/128) or 8-byte aligned. */
int64_t qgemv_mfma_codes(int32_t bits, int32_t group);

/* Free the host-side handle (never touches device memory). NULL is a no-op. */
void qgemv_destroy(qgemv_t h);

/* y[i][j] for i < m, j < n, contiguous (row stride n).
 *   x  bf16 bits [m][k] device, 16-byte aligned.
 *   m  window rows: 0..16 (decode windows), and on a matrix-core
 *      (QGEMV_ARITH_MFMA or _WIDE) handle up to QGEMV_MAX_PROMPT = 65
 *      (prompt windows: P788 keeps a row's bits in every window of 1-65
 *      rows in prompt).  m == 0 launches
 *      nothing and returns QGEMV_OK.  QGEMV_ARITH_DOT: a window whose staged
 *      activations exceed the LDS of one block (m*k*2.125 bytes > 152 KiB)
 *      is refused with QGEMV_E_WINDOW.  Matrix-core forms: a window above 16
 *      rows, or one too wide for the LDS, runs as passes of fewer rows (the
 *      weights are read once per pass); each row's bits are those of the
 *      row alone.
 *   y  fp32 [m][n] device, 4-byte aligned, must not overlap x or weights.
 *   epi QGEMV_EPI_NONE or QGEMV_EPI_RELU2.
 *   stream  hipStream_t (NULL = the null stream).
 * Refused on a handle with n_experts > 1 (QGEMV_E_ARG): describe a single
 * expert with its own qgemv_create over the expert's offset pointers. */
int qgemv_run(qgemv_t h, const uint16_t* x, int32_t m, float* y, int32_t epi, void* stream);

/* As qgemv_run, but writes y[i*ldy + j] for j < n only; every other element
 * of y is left untouched.  ldy < n is refused (QGEMV_E_STRIDE).  One member
 * (run) of a fused stack writes its columns into the stack output by
 * passing y + first_column and the stack's ldy.  Each row's bits equal
 * qgemv_run's. */
int qgemv_run_strided(qgemv_t h, const uint16_t* x, int32_t m, float* y, int64_t ldy,
                      int32_t epi, void* stream);

/* Indexed expert slots: y[(i*slots + s)*n + j] = epi(row i times expert
 * idx[i*slots + s]) for i < m, s < slots, j < n.
 *   idx  int32 [m][slots] device.  Each value must lie in [0, n_experts):
 *        a precondition on the caller (the values are read on the device
 *        only); values outside it write nothing for that slot.
 *   slots  0..64; slots == 0 or m == 0 launches nothing.
 * Each expert named in idx is read once per call; each (i, s) output's bits
 * equal qgemv_run on that expert's single-expert handle with row i. */
int qgemv_run_indexed(qgemv_t h, const uint16_t* x, int32_t m, const int32_t* idx,
                      int32_t slots, float* y, int32_t epi, void* stream);

/* Checked mode of the indexed calls, for tests and debugging, never for the
 * decode path: the pages read routing tables on the host and refuse a bad
 * one by name ("fail closed", P774 "What this changes", item 3).  Copies
 * idx [m][slots] (device) to the host, which waits for `stream` (this is
 * the one call that synchronises), and returns QGEMV_E_INDEX if any value
 * lies outside [0, n_experts) of h, else QGEMV_OK.  m in 0..16 and slots in
 * 0..64 as for qgemv_run_indexed (QGEMV_E_WINDOW / QGEMV_E_ARG otherwise);
 * QGEMV_E_HIP if the copy fails.  Launches nothing. */
int qgemv_check_indices(qgemv_t h, const int32_t* idx, int32_t m, int32_t slots, void* stream);

/* ---- gate/up pairs ------------------------------------------------------
 * The fused gate/up of a gated MLP or expert ("experts gate/up (through
 * silu)" and "the fused gate/up", P788 "tf-flashnext-widths"; one kernel
 * reads both, so gate and up must share a width, P774 "What this changes"):
 *   y[i][j] = silu(g) * u,   g = row j of `gate` times x[i],
 *                            u = row j of `up`   times x[i],
 *   silu(g) = g / (1 + exp(-g)) in fp32 (the device library's expf).
 * g and u have exactly the bits qgemv_run gives each handle; one dispatch
 * reads both matrices.  gate and up: matrix-core handles of one form
 * (QGEMV_ARITH_MFMA or _WIDE) and of equal bits, group, n, k and
 * n_experts (QGEMV_E_NOKERNEL for another form,
 * QGEMV_E_SHAPE for unequal shapes).  Windows, strides, alignment, aliasing
 * and refusals as qgemv_run_strided (m up to QGEMV_MAX_PROMPT) and
 * qgemv_run_indexed (the same expert of both stacks for each slot). */
int qgemv_run_gateup(qgemv_t gate, qgemv_t up, const uint16_t* x, int32_t m, float* y, int64_t ldy,
                     void* stream);
int qgemv_run_gateup_indexed(qgemv_t gate, qgemv_t up, const uint16_t* x, int32_t m, const int32_t* idx,
                             int32_t slots, float* y, void* stream);

/* ---- exact widen / regroup ----------------------------------------------
 * Members of one projection stored at different widths can be brought to a
 * single width: the largest bit count and the smallest group among them
 * (P788, the commit that adds widen.zig, "...tables repeated for a smaller
 * group").
 * qgemv_common_width: that width of `count` members (bits and groups as in
 *   qgemv_desc; QGEMV_E_BITS / QGEMV_E_GROUP for values the kernels do not
 *   run, QGEMV_E_ARG for count < 1).  Host only.
 * qgemv_widen: src's codes re-cut at bits_out bits (the same integer codes,
 *   low code first) and each group's scale and bias repeated for the
 *   src->group / group_out groups it splits into, so every dequantized value
 *   scale * q + bias is unchanged, bit for bit.  src is admitted as
 *   qgemv_create admits it; an expert stack widens row for row.  Output
 *   arrays (device, caller-owned): w_out uint32 [E][N][K*bits_out/32]
 *   16-byte aligned, scales_out and biases_out bf16 [E][N][K/group_out].
 *   Narrowing (bits_out < src->bits) is refused with QGEMV_E_BITS, a group
 *   that does not divide the source group with QGEMV_E_GROUP, outputs that
 *   overlap the source or each other with QGEMV_E_ALIAS.  Enqueued on
 *   `stream`; the same width and group copy the arrays as they are.  A
 *   fused projection's members widen one call each into consecutive rows of
 *   one output, keeping each member's values in order. */
int qgemv_common_width(const int32_t* bits, const int32_t* groups, int32_t count, int32_t* bits_out,
                       int32_t* group_out);
int qgemv_widen(const qgemv_desc* src, int32_t bits_out, int32_t group_out, uint32_t* w_out, uint16_t* scales_out,
                uint16_t* biases_out, void* stream);

/* Test hook: the kernels' own unpack of expert `expert` into codes[n][k]
 * (uint8, device, n*k bytes): each code is cut and converted exactly as the
 * product kernels do it, then written back as an integer. */
int qgemv_debug_unpack(qgemv_t h, int32_t expert, uint8_t* codes, void* stream);

/* Name of a status code ("QGEMV_E_STRIDE", ...); never NULL. */
const char* qgemv_strerror(int status);

/* ---- fused stacks ------------------------------------------------------
 * A fused projection is a set of runs sharing one input: each run is one
 * matrix of one width and group, and its members (consecutive row ranges of
 * the run) write their own columns of one output row of ldy columns, with no
 * scratch copy.  qgemv_stack_run computes every run in ONE dispatch per
 * arithmetic form present (each run takes qgemv_create's choice, so one
 * dispatch unless some run's shape rules out the matrix cores); each
 * member's columns are bit for bit what qgemv_run_strided of that run's own
 * handle writes there (same kernels, same arithmetic).  Columns outside every
 * member are left untouched.
 * Sources, on "Qwen3.8-Flash-Next faster kernels in Zig engine - #788":
 * commit "...row kernel at every MLX width" (callStrided: one member of a
 * fused stack writes its columns straight into the stack output), and on
 * "Qwen3.8-Flash-Next support for oQ in Zig engine - #774", "What this
 * changes" items 2-3 (runs grouped by width, placed at their members'
 * columns through a column map; oQ4e's ragged 6192/48 runs). */
#define QGEMV_MAX_RUNS 8
#define QGEMV_MAX_MEMBERS 4

typedef struct qgemv_run_spec {
  qgemv_desc w;                            /* the run's weights; w.n_experts must be 1 */
  int32_t n_members;                       /* 1..QGEMV_MAX_MEMBERS */
  int64_t member_rows[QGEMV_MAX_MEMBERS];  /* rows of each member in the run's row order; sum = w.n */
  int64_t member_cols[QGEMV_MAX_MEMBERS];  /* first output column of each member */
} qgemv_run_spec;

typedef struct qgemv_stack* qgemv_stack_t;

/* Validate every run as qgemv_create does (its status is returned as is),
 * then: 1 <= n_runs <= QGEMV_MAX_RUNS, every run has the same k (else
 * QGEMV_E_SHAPE), member rows are >= 1 and sum to the run's n (QGEMV_E_SHAPE),
 * every member's columns lie in [0, ldy) (QGEMV_E_STRIDE), no two members
 * share a column (QGEMV_E_ALIAS), and every dot-form run has k a whole
 * number of 16-lane chunks (QGEMV_E_NOKERNEL otherwise).  Borrows the weight
 * pointers; makes no HIP call. */
int qgemv_stack_create(const qgemv_run_spec* runs, int32_t n_runs, int64_t ldy, qgemv_stack_t* out);

/* y[i*ldy + c] for every member column c and window row i < m, in one
 * dispatch; x bf16 [m][k]; m 0..16 (0: nothing launched); epi as qgemv_run.
 * y must not overlap x or any run's weights (QGEMV_E_ALIAS). */
int qgemv_stack_run(qgemv_stack_t s, const uint16_t* x, int32_t m, float* y, int32_t epi, void* stream);

/* Free the host-side stack handle. NULL is a no-op. */
void qgemv_stack_destroy(qgemv_stack_t s);

/* Launch geometry fixed at create (for tests and reports):
 *   out[0] lanes per output column, out[1] output columns per wave,
 *   out[2] codes per lane chunk, out[3] threads per block of a 1-row
 *   window, out[4] output columns per block tile of a 1-row window (the
 *   K split of a matrix-core handle spreads each column over that many
 *   waves), out[5] compute units seen.   */
int qgemv_query(qgemv_t h, int64_t out[6]);

#ifdef __cplusplus
}
#endif

#endif /* QGEMV_H */
