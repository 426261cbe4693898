// Descriptor structs shared by the host planner and the gfx950 kernels.
//
// All tables live in the caller's device state buffer ("arena").  A pointer
// the kernels dereference is (base table entry) + (element offset): base 0 is
// the arena itself, bases 1..n are the gradients of the n tensors of this
// call, bases n+1..2n their weights.  The gradient/weight pointers change per
// call and are refreshed by a small host-to-device copy; everything else is
// built once by the planner.
#pragma once
#include <cstdint>

namespace shampoo {

constexpr int kMaxNewtonP = 8;

// One C = op(A) * op(B) problem of the batched GEMM kernel (row-major
// operands; op(X) = X or X^T).  The kernel covers it with 128x128 tiles.
struct GemmTask {
    int64_t a_off, b_off, c_off;  // element offsets from their bases
    int32_t a_base, b_base, c_base;
    int32_t M, N, K;              // op(A) is M x K, op(B) is K x N
    int32_t lda, ldb, ldc;
    int32_t trans;                // bit 0: op(A) = A^T, bit 1: op(B) = B^T, bits 2/3:
                                  // Newton operand on A/B, bit 4: upper tiles only
                                  // (symmetric C), bit 5: mirror off-diagonal tiles
    int32_t tiles_n;              // ceil(N / 128)
    int32_t factor;               // gating factor id (-1: always run)
    int32_t norm_slot;            // first slot of per-tile ||C||^2 partials, -1: none
    int32_t kb;                   // first k of the product (a split-K part sums k in [kb, K))
};

// One Shampoo block of at most 128 x 128 for the fused statistics kernel.
struct GramJob {
    int64_t g_off;        // element offset of G_b in its base (the tensor's gradient)
    int64_t l_off, r_off; // fp64 statistics (arena elements of 8 bytes)
    int32_t g_base;       // base index of the gradient
    int32_t ldg;          // tensor row length
    int32_t mb, nb;       // block shape
    int32_t ld_l, ld_r;   // leading dims of L and R
};

// One Shampoo block of at most 128 x 128 for the fused apply kernel.
struct ApplyJob {
    int64_t g_off;          // G_b in its base (the tensor's gradient)
    int64_t a_off, d_off;   // Adagrad accumulator and D blocks (arena floats)
    int64_t pl_off, pr_off; // fp32 roots (arena floats)
    int32_t g_base;         // gradient base index
    int32_t ldg;            // tensor row length (leading dim of G, a and D)
    int32_t mb, nb;
    int32_t ld_l, ld_r;
    int32_t slot_a, slot_d; // ||A_b||^2 and ||D_b||^2 slots
    int64_t m_off;          // momentum block (arena floats), used when fuse is set
    int32_t w_base;         // weight base index, used when fuse is set
    int32_t fuse;           // 1: graft, momentum and weight update in the same kernel
};

// One Shampoo block of at most 128 x 128 for the fused step kernel
// (statistics and apply together, on steps without a root pass).
struct StepJob {
    ApplyJob ap;
    int64_t l_off, r_off;   // fp64 statistics (arena elements of 8 bytes)
};

// One contiguous copy inside the state buffer (bytes, multiples of 16).
struct CopyJob {
    int64_t src, dst, bytes;
};

// Sum of the split-K partial products of one large statistic (one-sided
// preconditioning): S <- beta S + alpha sum_c part_c, over the upper
// triangle, written to both triangles.  part_c holds the upper 128 x 128
// tiles of chunk c's product (leading dim ld, ld * ld doubles apart).
struct SymReduceJob {
    int64_t part_off;   // first partial (arena elements of 8 bytes)
    int64_t s_off;      // statistic (arena elements of 8 bytes)
    int32_t nparts;     // number of partials
    int32_t dim, ld;
    int32_t tiles;      // 32 x 32 tiles per side: ceil(dim / 32)
};

// One symmetric product of the batched Newton chain that was split over k:
// C = sum of its nparts partial products (upper 128 x 128 tiles of each), in
// part order, written to both triangles of C.
struct SplitSumJob {
    int64_t part_off;   // first partial (elements of the chain's type from the arena base)
    int64_t c_off;      // destination C (same units)
    int32_t nparts;     // partials, ld * ld elements apart
    int32_t ld;         // padded dimension (a multiple of 32)
    int32_t tiles;      // ld / 32
    int32_t gate;       // gating id (-1: always run)
};

// One C = A B^T problem of the split-precision (bf16x3) GEMM kernel: A is
// M x K and B is N x K, both row-major with k contiguous (fp32), C is M x N
// fp32.  Used for the two products of the apply, D = P_L (P_R G^T)^T: the
// first product's B is the gradient block, whose elements the kernel can
// also take through the Adagrad accumulator on the way.
struct NtTask {
    int64_t a_off, b_off, c_off;  // element offsets from their bases
    int32_t a_base, b_base, c_base;
    int32_t M, N, K;
    int32_t lda, ldb, ldc;
    int32_t tiles_n;              // ceil(N / 128)
    int32_t norm_slot;            // first slot of per-tile ||C||^2 partials, -1: none
    int64_t acc_off;              // >= 0: Adagrad accumulator of B's elements (arena floats,
                                  // leading dim ldb), updated by the tiles of row 0
    int32_t acc_slot;             // first ||A||^2 partial slot (one per tile column)
    int32_t pad_;
};

// A tile of the batched GEMM launch: which task and which 128x128 tile.
struct TileRef {
    int32_t task;
    int32_t tile;
};

// One symmetric matrix for the Lanczos kernel.
struct LanczosJob {
    int64_t off;      // element offset of the matrix in the arena (fp64 statistics or fp32 root)
    int32_t n;        // real dimension
    int32_t ld;       // leading dimension
    int32_t factor;   // factor id (diagnostics record)
    int32_t p;        // root exponent of the factor (mode 1: kappa of S from that of P)
};

// Per-factor job of the Newton init / commit kernels.
struct FactorJob {
    int64_t s_off;    // fp64 statistics (arena elements of 8 bytes)
    int64_t p_off;    // fp32 root
    int64_t p64_off;  // fp64 root (arena element offset in doubles), -1 none
    int64_t x_off;    // scratch X (elements of the scratch type)
    int64_t m_off;    // scratch M
    int32_t n;        // real dimension
    int32_t ld;       // padded dimension (leading dim of every matrix)
    int32_t factor;
    int32_t pad_;
};

// One class (padded dimension, root exponent) of the gated fp64 Newton chain.
// The factors whose precision flag routes them to fp64 are packed, in class
// order, into the leading slots of the class, so that the chain's launches
// run on the routed factors only; slot k's scratch sits at place k mod cap
// of its chunk.
struct CompactClass {
    int32_t first;   // first entry of the class in the template, slot-job and slot-flag arrays
    int32_t n;       // factors (and slots) in the class
    int32_t cap;     // slots per scratch chunk
    int32_t pad_;
    int64_t mat;     // ld * ld (six scratch matrices per slot)
};

// A run of rows of one dense tensor for the elementwise kernels.
struct RowChunk {
    int32_t tensor;       // tensor index (its gradient/weight base = 1 + tensor, 1 + n + tensor)
    int32_t mode;         // 0: Shampoo (graft), 1: dense Adagrad
    int32_t row0, nrows;
    int32_t cols;
    int32_t block_size;
    int32_t first_block;  // Shampoo: first block of the tensor
    int32_t nbc;          // Shampoo: blocks per block-row
    int64_t a_off;        // Adagrad accumulator (arena element offset)
    int64_t m_off;        // momentum
    int64_t d_off;        // preconditioned gradient D (Shampoo only)
};

// A run of rows inside one Shampoo block for the Adagrad/||A||^2 kernel.
struct BlockChunk {
    int32_t tensor, block;
    int32_t row0, nrows;  // rows within the tensor
    int32_t col0, ncols;  // columns of the block
    int32_t cols;         // tensor row length
    int32_t slot;         // partial ||A||^2 slot
    int64_t a_off;        // accumulator of the tensor
};

// Per-block reduction ranges for the graft scale.
struct BlockNorms {
    int32_t a_first, a_count;  // partial ||A_b||^2 slots
    int32_t d_first, d_count;  // partial ||D_b||^2 slots
    int32_t block;             // graft scale index (the block)
    int32_t pad_;
};

// One sparse table of one call.
struct SparseJob {
    int64_t rows_ptr;     // const int32_t*
    int64_t grads_ptr;    // const float*
    int64_t w_ptr;        // float*
    int64_t a_off;        // accumulator (arena elements)
    int64_t n_rows;
    int64_t first_item;   // prefix over jobs of n_rows * (cols / 4 or cols)
    int64_t table_rows;   // rows of the table (row ids outside [0, table_rows) are skipped)
    int32_t cols;
    int32_t vec;          // 1: float4 path
};

// One sparse-row table with one-sided preconditioning, for one call: its
// listed rows are processed in chunks of chunk_rows rows, one workgroup each
// (chunks of all tables numbered consecutively from first_chunk).
struct SosJob {
    int64_t rows_ptr;     // const int32_t*: listed row ids (distinct)
    int64_t grads_ptr;    // const float*: n_rows x cols row gradients g
    int64_t w_ptr;        // float*: the table's weights
    int64_t a_off;        // Adagrad accumulator of the table (arena floats)
    int64_t d_off;        // D = g P, n_rows x cols (arena floats)
    int64_t n_rows;
    int64_t table_rows;   // row ids outside [0, table_rows) are skipped
    int32_t cols;
    int32_t chunk_rows;
    int32_t first_chunk;
    int32_t slot_a;       // first ||A||^2 partial slot (one per chunk)
    int32_t block;        // graft scale index (the table's block)
    int32_t vec;          // 1: float4 path
};

// Device-side copy of the public diagnostics record (same layout).
struct FactorDiag {
    double lambda_max, eps, kappa_est, residual;
    int32_t block, side, dim, status;
    int32_t iters, reserved_;
};

}  // namespace shampoo
