// Launch interface of the gfx950 kernels (host side).
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

#include "common.hpp"

namespace shampoo {

enum : int {
    SHAMPOO_FACTOR_NONFINITE_INPUT_ = 1,
    SHAMPOO_FACTOR_NONFINITE_ROOT_ = 2,
    SHAMPOO_FACTOR_RESIDUAL_HIGH_ = 4,
    SHAMPOO_FACTOR_FP64_ = 8,
    SHAMPOO_FACTOR_ZERO_ = 16,
};

enum : int { EPI_STORE = 0, EPI_AXPBY = 1 };

struct GemmArgs {
    int epi;              // EPI_STORE or EPI_AXPBY
    double alpha, beta;   // C = alpha acc (+ beta C)
    double xc1, xc2;      // Newton operand transform c1 I + c2 X (trans bits 2/3)
    const int32_t* gate;  // per-factor precision flags, or null
    int32_t gate_val;     // run only tasks whose factor has this flag
    double* norms;        // per-tile ||C||^2 partials (tasks with norm_slot >= 0)
    // fp64 store launches only: > 0 runs that many workgroups over a tile
    // table sorted by gating id (a workgroup stops at its first gated tile,
    // as every later one is gated too); ntiles is the table's length.  With
    // chain > 1 the table holds groups of `chain` one-tile products that one
    // workgroup runs in order, each reading what the previous ones wrote.
    int32_t persist;
    int32_t ntiles;
    int32_t chain;
};

// Lanczos on at most this many factors > 128 splits each step's product over
// many workgroups (a work record of kLzWork doubles per factor).
constexpr int kLanczosSplitMax = 32;
constexpr int kLzWork = 3 * 1024 + 2 * 64 + 4;

// Relative Ritz residual at which the adaptive Lanczos stops: the estimate of
// lambda_max is then within this fraction of an eigenvalue.
constexpr double kLanczosTol = 5e-5;

struct LanczosArgs {
    int steps;            // at most this many steps
    double tol;           // > 0: stop once the top Ritz residual <= tol theta
    int mode;             // 0: statistics (lambda_max, eps), 1: roots (kappa estimate)
    int auto_route;       // mode 1: set prec flags from the kappa estimate
    int route_all_fp64;   // mode 0: initial prec flag value
    double eps_rel;
    double threshold;
    FactorDiag* diag;
    int32_t* prec;
    double* work;         // factors > 128: split Lanczos work records (kLanczosSplitMax of them)
    int max_n;            // factors > 128: the largest dimension among the jobs (0: up to 1024)
};

struct NewtonArgs {
    int p;
    int is_fp64;
    const int32_t* gate;
    int32_t gate_val;
    int iters;                 // iterations run (recorded in the diagnostics)
    double xc1, xc2;           // the first step's T = xc1 I + xc2 M (the start forms X_1)
    unsigned long long* chk;   // per factor: [2f] max |M - I| (bits), [2f + 1] non-finite flag
};

struct FusedArgs {          // fused fp32 root of factors up to 128
    int p, iters;
    int steps_s, steps_p;   // Lanczos steps on S (lambda_max) and on the root (kappa)
    double lz_tol;          // > 0: Lanczos on S stops once its Ritz residual <= lz_tol theta
    int auto_route;         // set prec flags from the kappa estimate
    double eps_rel, threshold;
    float tol;              // > 0: stop one step after ||M - I||_F < tol (at most iters)
};

struct NtArgs {
    double* norms;        // per-tile ||C||^2 partials (tasks with norm_slot >= 0)
    double* partA;        // ||A||^2 partials of the Adagrad-fused tasks
    float* arena;         // base of the accumulator offsets
    float delta;          // graft epsilon of A = G / (sqrt(a) + delta)
};

struct UpdateArgs {
    float beta1, lr, delta;
};

// Static device scratch of the allocation-free root pass
// (shampoo_compute_inverse_roots_noalloc): the batched coupled-Newton iterates,
// six ld x ld matrices per factor slot; one fp64 slot of the largest factor
// (ld 1024) takes 48 MiB.
constexpr size_t kNoallocScratchBytes = size_t(64) << 20;
// Its address on the current device (asked of the runtime once per device).
hipError_t noalloc_scratch_ptr(void** out);

// role: 0 Newton products, 1 / 2 the first / second product of the apply
// (the same kernel; the role only names the instantiation for profilers)
hipError_t launch_gemm_f32(const GemmTask* tasks, const TileRef* tiles, int ntiles,
                           const uint64_t* bases, const GemmArgs& a, hipStream_t s, int role = 0);
// The split-precision (bf16x3) C = A B^T products of the apply; adagrad:
// tasks with acc_off >= 0 also run the Adagrad pass over B's elements.
hipError_t launch_gemm_nt3(const NtTask* tasks, const TileRef* tiles, int ntiles,
                           const uint64_t* bases, const NtArgs& a, bool adagrad, hipStream_t s);
hipError_t launch_gemm_f64(const GemmTask* tasks, const TileRef* tiles, int ntiles,
                           const uint64_t* bases, const GemmArgs& a, hipStream_t s);
hipError_t launch_gemm_f64_from_f32(const GemmTask* tasks, const TileRef* tiles, int ntiles,
                                    const uint64_t* bases, const GemmArgs& a, hipStream_t s);
hipError_t launch_gram128(const GramJob* jobs, int njobs, const uint64_t* bases, double* stats,
                          double alpha, double beta, hipStream_t s);
// Blocks <= 128 of a step without a root pass; with nfold > 0 the launch also
// runs the dense-Adagrad row chunks `fold` (workgroups after the blocks).
hipError_t launch_step128(const StepJob* jobs, int njobs, const RowChunk* fold, int nfold,
                          int n_tensors, const uint64_t* bases, float* arena, double alpha, double beta,
                          float delta, double* partA, double* partD, const UpdateArgs& ua,
                          hipStream_t s);
hipError_t launch_lanczos(const LanczosJob* jobs, int njobs, const void* arena, bool fp64_matrix,
                          bool big, const LanczosArgs& a, hipStream_t s);
// Sums the split-K parts of symmetric Newton products (one workgroup per
// 32 x 32 tile pair) into both triangles of their destinations.
hipError_t launch_split_sum(bool fp64, const SplitSumJob* jobs, const TileRef* tiles, int ntiles,
                            void* arena, const int32_t* gate, int gate_val, hipStream_t s);
// Packs the factors of each class routed to fp64 (flag gate_val) into the
// class's leading slots: slot jobs and slot flags (one workgroup per class).
hipError_t launch_route_compact(const CompactClass* cls, int ncls, const FactorJob* tmpl,
                                const int32_t* prec, int gate_val, FactorJob* slots, int32_t* live,
                                hipStream_t s);
// Newton start and finish, one workgroup per 32 x 32 tile of every factor of
// a chunk (factors of leading dimension ld).  The finish takes X from the
// buffer set at `scratch` and the last M formed from the one at `scratch_m`.
hipError_t launch_newton_init(bool fp64, const FactorJob* jobs, int njobs, int ld,
                              const double* stats, void* scratch, const FactorDiag* diag,
                              const NewtonArgs& a, hipStream_t s);
hipError_t launch_newton_commit(bool fp64, const FactorJob* jobs, int njobs, int ld, float* arena,
                                const void* scratch, const void* scratch_m, FactorDiag* diag,
                                const NewtonArgs& a, hipStream_t s);
hipError_t launch_newton128(const FactorJob* jobs, int njobs, const double* stats, float* arena,
                            FactorDiag* diag, int32_t* prec, const FusedArgs& a, hipStream_t s);
hipError_t launch_apply128(const ApplyJob* jobs, int njobs, const uint64_t* bases, float* arena,
                           float delta, double* partA, double* partD, const UpdateArgs& ua,
                           hipStream_t s);
hipError_t launch_copy_jobs(const CopyJob* jobs, int njobs, unsigned char* arena, hipStream_t s);
hipError_t launch_sos_norm(const SosJob* jobs, int njobs, int nchunks, float* arena, float delta,
                           double* partA, hipStream_t s);
hipError_t launch_sos_update(const SosJob* jobs, int njobs, int nchunks, float* arena,
                             const float* scale, float lr, hipStream_t s);
hipError_t launch_sym_reduce(const SymReduceJob* jobs, const TileRef* tiles, int ntiles,
                             double* arena, double alpha, double beta, hipStream_t s);
hipError_t launch_set_identity(const FactorJob* jobs, int njobs, float* arena, hipStream_t s);
hipError_t launch_adagrad_norm(const BlockChunk* chunks, int nchunks, const uint64_t* bases,
                               float* arena, float delta, double* partA, hipStream_t s);
hipError_t launch_block_scale(const BlockNorms* bn, int nblocks, const double* partA,
                              const double* partD, float* scale, hipStream_t s);
hipError_t launch_update(const RowChunk* chunks, int nchunks, const uint64_t* bases, int n_tensors,
                         float* arena, const float* scale, const UpdateArgs& a, hipStream_t s);
hipError_t launch_sparse_rows(const SparseJob* jobs, int njobs, int64_t total, float* arena,
                              float lr, float delta, hipStream_t s);

}  // namespace shampoo
