// gfx950 kernels of the Shampoo step.
//
// Method: "Scalable Second Order Optimization for Deep Learning" (Anil et al.);
// Shampoo-at-scale podcast transcript, cues 6-16: per-dimension statistics
// L, R; their inverse fourth roots by coupled Newton iteration (fp64 where the
// statistics are ill-conditioned); the two-sided preconditioned multiply;
// Lemma-2 blocking.  Grafting, momentum and the Adagrad fallbacks are this
// library's configuration (not on the pages).
//
// Kernels:
//   k_gemm<T>        batched C = alpha op(A) op(B) (+ beta C), 128x128 tiles on
//                    MFMA (fp32: v_mfma_f32_32x32x2f32, fp64:
//                    v_mfma_f64_16x16x4f64), operands staged through LDS;
//                    optional on-the-fly Newton operand T = c1 I + c2 M and
//                    per-tile ||C||^2 partials.  Used for the statistics, the
//                    two-sided apply and the batched coupled-Newton chain.
//   k_lanczos        Krylov extreme-eigenvalue estimate per symmetric matrix.
//   k_newton_init<T> / k_newton_commit<T>  start and finish of the batched
//                    coupled-Newton iteration.
//   k_sym_reduce     fixed-order sum of split-K partial statistics (one-sided
//                    preconditioning of a large layer) into S, both triangles.
//   k_sos_norm / k_sos_update  sparse-row tables with one-sided
//                    preconditioning: accumulator and ||A||^2 over the listed
//                    rows; W_r -= lr s D_r on those rows.
//   k_adagrad_norm   a <- a + G*G on Shampoo blocks and ||A_b||^2 partials.
//   k_block_scale    graft factor ||A_b|| / ||D_b|| per block.
//   k_update         momentum and weight update (and dense Adagrad fallback).
//   k_sparse_rows    sparse-row Adagrad for embedding tables.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace shampoo {

// ---------------------------------------------------------------- helpers
// One DPP step on a double (both halves moved the same way; rows outside
// ROWM take 0).
template <int CTRL, int ROWM>
__device__ __forceinline__ double dpp_d(double v) {
    const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), CTRL, ROWM, 0xf, false);
    const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), CTRL, ROWM, 0xf, false);
    return __hiloint2double(hi, lo);
}
// Sum over the 64 lanes of a wave, returned to every lane; called with all
// lanes active.  DPP moves (no LDS): pairs and quads, rows of 16 by two
// rotations, then the row broadcasts 15 and 31 leave the total in lane 63,
// which is read out.  A fixed order, so the result is deterministic.
__device__ __forceinline__ double wave_sum(double v) {
    v += dpp_d<0xB1, 0xf>(v);    // quad_perm [1,0,3,2]
    v += dpp_d<0x4E, 0xf>(v);    // quad_perm [2,3,0,1]
    v += dpp_d<0x124, 0xf>(v);   // row_ror:4
    v += dpp_d<0x128, 0xf>(v);   // row_ror:8
    v += dpp_d<0x142, 0xa>(v);   // row_bcast:15 into rows 1 and 3
    v += dpp_d<0x143, 0xc>(v);   // row_bcast:31 into rows 2 and 3
    const int lo = __builtin_amdgcn_readlane(__double2loint(v), 63);
    const int hi = __builtin_amdgcn_readlane(__double2hiint(v), 63);
    return __hiloint2double(hi, lo);
}
__device__ __forceinline__ float wave_sum(float v) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
__device__ __forceinline__ double wave_max(double v) {
    for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o, 64));
    return v;
}

// Fixed-order block reduction over 256 threads (deterministic).
__device__ __forceinline__ double block_sum_256(double v, double* red) {
    v = wave_sum(v);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    return (red[0] + red[1]) + (red[2] + red[3]);
}
__device__ __forceinline__ double block_max_256(double v, double* red) {
    v = wave_max(v);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    return fmax(fmax(red[0], red[1]), fmax(red[2], red[3]));
}

// A pointer from the per-call pointer table, cast through the global address
// space so that the compiler emits global (not flat) memory instructions:
// flat loads also count against the LDS wait counter, so an LDS wait would
// stall on them.
template <typename T>
__device__ __forceinline__ T* global_ptr(uint64_t addr) {
    typedef __attribute__((address_space(1))) T gT;
    return (T*)reinterpret_cast<gT*>(addr);
}
template <typename T>
__device__ __forceinline__ T* base_ptr(const uint64_t* bases, int b, int64_t off) {
    return global_ptr<T>(bases[b]) + off;
}

// ============================================================ batched GEMM
template <typename T> struct GemmTraits;
template <> struct GemmTraits<float> {
    static constexpr int BK = 32;   // k per LDS stage
    static constexpr int VEC = 4;   // elements per 16-byte global load
    static constexpr int PADE = 4;  // LDS row padding (elements)
};
template <> struct GemmTraits<double> {
    static constexpr int BK = 16;
    static constexpr int VEC = 2;
    static constexpr int PADE = 2;
};

constexpr int BM = 128, BN = 128;

template <typename T> struct Vec16;
template <> struct Vec16<float> { using type = float4; };
template <> struct Vec16<double> { using type = double2; };

// Loads one BK-deep stage of op(X) (rows [r0, r0+128) x k [k0, k0+BK)) into
// registers, converting the stored type TI to the compute type T.  `kcontig`:
// X is stored with k contiguous (X[r*ld + k]); otherwise r contiguous
// (X[k*ld + r]).  Out-of-range elements are zero; a stage wholly in range
// takes a path without checks.  The optional transform (Newton operand) maps
// the value v at op-index (r, k) to c2 v + c1 [r == k], the diagonal term
// only on stages that meet the diagonal.
template <typename T, typename TI>
struct StageLoader {
    static constexpr int BK = GemmTraits<T>::BK;
    static constexpr int VEC = GemmTraits<T>::VEC;
    typedef TI vec_t __attribute__((ext_vector_type(VEC)));
    T v[4][VEC];
    int t;   // thread index (set per tile: see gemm_tile)

    __device__ __forceinline__ void load(const TI* __restrict__ X, int ld, bool kcontig,
                                         int r0, int k0, int R, int K, bool aligned,
                                         bool xf, T c1, T c2, int dk) {
        // uniform over the workgroup: the whole stage is in range (no checks),
        // and whether it meets the diagonal r == k
        const bool full = aligned && r0 + BM <= R && k0 + BK <= K;
        const bool dg = xf && k0 + dk < r0 + BM && r0 < k0 + dk + BK;
        if (kcontig) {
            // 8 threads x VEC cover BK along k; 32 rows per pass, 4 passes.
            const int kq = t & 7, rr = t >> 3;
            if (full) {
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const vec_t q = *reinterpret_cast<const vec_t*>(
                        X + (int64_t)(r0 + rr + 32 * p) * ld + k0 + kq * VEC);
#pragma unroll
                    for (int e = 0; e < VEC; ++e) v[p][e] = T(q[e]);
                }
            } else {
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const int r = r0 + rr + 32 * p;
                    const int k = k0 + kq * VEC;
                    if (aligned && r < R && k + VEC <= K) {
                        const vec_t q = *reinterpret_cast<const vec_t*>(X + (int64_t)r * ld + k);
#pragma unroll
                        for (int e = 0; e < VEC; ++e) v[p][e] = T(q[e]);
                    } else {
#pragma unroll
                        for (int e = 0; e < VEC; ++e)
                            v[p][e] = (r < R && k + e < K) ? T(X[(int64_t)r * ld + k + e]) : T(0);
                    }
                }
            }
            if (xf) {
#pragma unroll
                for (int p = 0; p < 4; ++p)
#pragma unroll
                    for (int e = 0; e < VEC; ++e) v[p][e] *= c2;
                if (dg) {
#pragma unroll
                    for (int p = 0; p < 4; ++p) {
                        const int r = r0 + rr + 32 * p;
                        const int k = k0 + kq * VEC;
#pragma unroll
                        for (int e = 0; e < VEC; ++e)
                            if (r == k + e + dk && r < R && k + e < K) v[p][e] += c1;
                    }
                }
            }
        } else {
            // RQ threads x VEC cover 128 rows; KR k-rows per pass, 4 passes.
            constexpr int RQ = BM / VEC;
            constexpr int KR = 256 / RQ;
            const int rq = t % RQ, kr = t / RQ;
            if (full) {
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const vec_t q = *reinterpret_cast<const vec_t*>(
                        X + (int64_t)(k0 + kr + KR * p) * ld + r0 + rq * VEC);
#pragma unroll
                    for (int e = 0; e < VEC; ++e) v[p][e] = T(q[e]);
                }
            } else {
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const int k = k0 + kr + KR * p;
                    const int r = r0 + rq * VEC;
                    if (aligned && k < K && r + VEC <= R) {
                        const vec_t q = *reinterpret_cast<const vec_t*>(X + (int64_t)k * ld + r);
#pragma unroll
                        for (int e = 0; e < VEC; ++e) v[p][e] = T(q[e]);
                    } else {
#pragma unroll
                        for (int e = 0; e < VEC; ++e)
                            v[p][e] = (k < K && r + e < R) ? T(X[(int64_t)k * ld + r + e]) : T(0);
                    }
                }
            }
            if (xf) {
#pragma unroll
                for (int p = 0; p < 4; ++p)
#pragma unroll
                    for (int e = 0; e < VEC; ++e) v[p][e] *= c2;
                if (dg) {
#pragma unroll
                    for (int p = 0; p < 4; ++p) {
                        const int k = k0 + kr + KR * p;
                        const int r = r0 + rq * VEC;
#pragma unroll
                        for (int e = 0; e < VEC; ++e)
                            if (r + e == k + dk && k < K && r + e < R) v[p][e] += c1;
                    }
                }
            }
        }
    }

    // LDS layout: S[k][r] with row pitch 128 + PADE (r contiguous).
    __device__ __forceinline__ void store(T* S, bool kcontig) const {
        constexpr int P = BM + GemmTraits<T>::PADE;
        if (kcontig) {
            const int kq = t & 7, rr = t >> 3;
#pragma unroll
            for (int p = 0; p < 4; ++p)
#pragma unroll
                for (int e = 0; e < VEC; ++e) S[(kq * VEC + e) * P + rr + 32 * p] = v[p][e];
        } else {
            constexpr int RQ = BM / VEC;
            constexpr int KR = 256 / RQ;
            const int rq = t % RQ, kr = t / RQ;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                typename Vec16<T>::type q;
                T* qs = reinterpret_cast<T*>(&q);
#pragma unroll
                for (int e = 0; e < VEC; ++e) qs[e] = v[p][e];
                *reinterpret_cast<typename Vec16<T>::type*>(&S[(kr + KR * p) * P + rq * VEC]) = q;
            }
        }
    }
};

// MFMA micro-kernels: each wave owns a 64x64 sub-tile of the 128x128 tile.
template <typename T> struct WaveTile;

template <> struct WaveTile<float> {
    // 2x2 tiles of 32x32 (v_mfma_f32_32x32x2f32: A lane l = A[l%32][l/32],
    // B lane l = B[l/32][l%32], C lane l reg v = C[8(v/4) + 4(l/32) + v%4][l%32]).
    typedef float acc_t __attribute__((ext_vector_type(16)));
    acc_t acc[2][2];
    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
    }
    // The operands of step kk + 2 are read from LDS before the products of
    // step kk are issued (the scheduling groups keep that order), so a read's
    // latency overlaps four MFMAs instead of stalling the wave.
    // Ap, Bp: the wave's 64 rows of op(A) and 64 columns of op(B) in the
    // stages (layout [k][P]).
    __device__ __forceinline__ void compute(const float* Ap, const float* Bp) {
        constexpr int P = BM + GemmTraits<float>::PADE;
        constexpr int BK = GemmTraits<float>::BK;
        const int lane = threadIdx.x & 63;
        const int h = lane >> 5, c = lane & 31;
        float a[2], b[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) a[i] = Ap[h * P + i * 32 + c];
#pragma unroll
        for (int j = 0; j < 2; ++j) b[j] = Bp[h * P + j * 32 + c];
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // 2 LDS reads
#pragma unroll
        for (int kk = 0; kk < BK; kk += 2) {
            float an[2], bn[2];
            if (kk + 2 < BK) {
#pragma unroll
                for (int i = 0; i < 2; ++i) an[i] = Ap[(kk + 2 + h) * P + i * 32 + c];
#pragma unroll
                for (int j = 0; j < 2; ++j) bn[j] = Bp[(kk + 2 + h) * P + j * 32 + c];
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], b[j], acc[i][j], 0, 0, 0);
            if (kk + 2 < BK) {
                a[0] = an[0]; a[1] = an[1]; b[0] = bn[0]; b[1] = bn[1];
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // next step's reads
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);       // then 4 MFMAs
        }
    }
    // accumulator value idx = (2 i + j) 16 + v and its place (r, c) in the tile
    static constexpr int NV = 64;
    __device__ __forceinline__ float get(int idx, int wm, int wn, int& r, int& c) const {
        const int lane = threadIdx.x & 63;
        const int i = idx >> 5, j = (idx >> 4) & 1, v = idx & 15;
        r = wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        c = wn * 64 + j * 32 + (lane & 31);
        return acc[i][j][v];
    }
    // alpha times the wave's sub-tile, transposed, at Ct (Ct[c * ldc + r]):
    // registers v = 4q .. 4q + 3 of a lane are four consecutive rows r, so
    // each lane stores 16 bytes per group (one row of the transpose)
    __device__ __forceinline__ void store_transposed(float* Ct, int ldc, int wm, int wn,
                                                     float alpha) const {
        const int lane = threadIdx.x & 63;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int r = wm * 64 + i * 32 + 8 * q + 4 * (lane >> 5);
                    const int c = wn * 64 + j * 32 + (lane & 31);
                    const float4 x = make_float4(alpha * acc[i][j][4 * q], alpha * acc[i][j][4 * q + 1],
                                                 alpha * acc[i][j][4 * q + 2],
                                                 alpha * acc[i][j][4 * q + 3]);
                    *reinterpret_cast<float4*>(Ct + (int64_t)c * ldc + r) = x;
                }
    }
};

template <> struct WaveTile<double> {
    // 4x4 tiles of 16x16 (v_mfma_f64_16x16x4f64: A lane l = A[l%16][l/16],
    // B lane l = B[l/16][l%16], C lane l reg v = C[l/16 + 4v][l%16] -- note
    // the row order differs from the fp32 16x16x4 form).
    typedef double acc_t __attribute__((ext_vector_type(4)));
    acc_t acc[4][4];
    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[i][j][v] = 0.0;
    }
    __device__ __forceinline__ void compute(const double* Ap, const double* Bp) {
        constexpr int P = BM + GemmTraits<double>::PADE;
        const int lane = threadIdx.x & 63;
        const int g = lane >> 4, c = lane & 15;
#pragma unroll
        for (int kk = 0; kk < GemmTraits<double>::BK; kk += 4) {
            double a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = Ap[(kk + g) * P + i * 16 + c];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = Bp[(kk + g) * P + j * 16 + c];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], b[j], acc[i][j], 0, 0, 0);
        }
    }
    // the same from fp32 stages of BK = 32 (fp32 operands: each value is
    // converted to fp64 as it is read, exactly), the wave's 64 rows of op(A)
    // and 64 columns of op(B) at Ap and Bp (stage layout [k][P])
    // (with the next step's operands read from LDS before this step's 16
    // products, as in the fp32 tile)
    __device__ __forceinline__ void compute_f32(const float* Ap, const float* Bp) {
        constexpr int P = BM + GemmTraits<float>::PADE;
        constexpr int BK = GemmTraits<float>::BK;
        const int lane = threadIdx.x & 63;
        const int g = lane >> 4, c = lane & 15;
        float a[4], b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = Ap[g * P + i * 16 + c];
#pragma unroll
        for (int j = 0; j < 4; ++j) b[j] = Bp[g * P + j * 16 + c];
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
        for (int kk = 0; kk < BK; kk += 4) {
            float an[4], bn[4];
            if (kk + 4 < BK) {
#pragma unroll
                for (int i = 0; i < 4; ++i) an[i] = Ap[(kk + 4 + g) * P + i * 16 + c];
#pragma unroll
                for (int j = 0; j < 4; ++j) bn[j] = Bp[(kk + 4 + g) * P + j * 16 + c];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)a[i], (double)b[j], acc[i][j],
                                                                     0, 0, 0);
            if (kk + 4 < BK) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    a[i] = an[i];
                    b[i] = bn[i];
                }
                __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
        }
    }
    // accumulator value idx = (4 i + j) 4 + v and its place (r, c) in the tile
    static constexpr int NV = 64;
    __device__ __forceinline__ double get(int idx, int wm, int wn, int& r, int& c) const {
        const int lane = threadIdx.x & 63;
        const int i = idx >> 4, j = (idx >> 2) & 3, v = idx & 3;
        r = wm * 64 + i * 16 + (lane >> 4) + 4 * v;
        c = wn * 64 + j * 16 + (lane & 15);
        return acc[i][j][v];
    }
};

// C (type T) = alpha op(A) op(B) (+ beta C); A, B stored as TA, TB and
// converted to T on the way into LDS (fp32 gradients into an fp64 product are
// exact: fp32 x fp32 fits the fp64 mantissa).
// One tile of a batched-GEMM launch (entry e of the tile table); false if
// its task is gated off.
// fp64 products of fp32 operands (the statistics) stage their operands in
// LDS as fp32, 32 deep, and convert them as they are read: half the LDS bytes
// and barriers per k of fp64 stages.
template <typename T, typename TA, typename TB>
constexpr bool kStageF32 = sizeof(T) == 8 && sizeof(TA) == 4 && sizeof(TB) == 4;

template <typename T, typename TA, typename TB, bool AXPBY, bool XF, bool PERSIST>
__device__ __forceinline__ bool gemm_tile(int e, const GemmTask* __restrict__ tasks,
                                          const TileRef* __restrict__ tiles,
                                          const uint64_t* __restrict__ bases, const GemmArgs& args,
                                          void* As_, void* Bs_, double* red) {
    constexpr bool F32S = kStageF32<T, TA, TB>;
    using S = typename std::conditional<F32S, float, T>::type;   // staged type
    S* As = static_cast<S*>(As_);
    S* Bs = static_cast<S*>(Bs_);
    constexpr int BK = GemmTraits<S>::BK;
    const TileRef tr = tiles[e];
    const GemmTask tk = tasks[tr.task];
    if (args.gate && tk.factor >= 0 && args.gate[tk.factor] != args.gate_val) return false;

    // symmetric squares (trans bit 6: the statistics, and Newton products of
    // one operand with itself): a negative tile index -1 - q stands for group
    // q of the diagonal band (below), staged as tile (t0, t0 + 1)
    const bool band = (F32S || XF) && tr.tile < 0;
    const int q = -1 - tr.tile, t0 = (4 * q) / 3;
    const int ti = band ? t0 : tr.tile / tk.tiles_n, tj = band ? t0 + 1 : tr.tile % tk.tiles_n;
    const int i0 = ti * BM, j0 = tj * BN;
    const TA* A = base_ptr<TA>(bases, tk.a_base, tk.a_off);
    const TB* B = base_ptr<TB>(bases, tk.b_base, tk.b_off);
    T* C = base_ptr<T>(bases, tk.c_base, tk.c_off);
    const bool ta = tk.trans & 1, tb = (tk.trans >> 1) & 1;
    // the Newton operand transform, compiled only where XF
    const bool xa = XF && ((tk.trans >> 2) & 1), xb = XF && ((tk.trans >> 3) & 1);
    // op(A) = A: A[i][k] has k contiguous.  op(A) = A^T: A[k][i], i contiguous.
    const bool a_kc = !ta;
    // op(B)[k][j]: B^T stored B[j][k] -> k contiguous; B stored B[k][j] -> j contiguous.
    const bool b_kc = tb;
    constexpr int VEC = GemmTraits<S>::VEC;
    const bool a_al = ((reinterpret_cast<uintptr_t>(A) % (VEC * sizeof(TA))) == 0) && (tk.lda % VEC == 0);
    const bool b_al = ((reinterpret_cast<uintptr_t>(B) % (VEC * sizeof(TB))) == 0) && (tk.ldb % VEC == 0);
    const S c1 = S(args.xc1), c2 = S(args.xc2);

    // the wave index as a scalar: branches on it are uniform to the compiler
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = w >> 1, wn = w & 1;
    // The wave's operand slots: 64-row halves of the stages, 0 and 1 of A's,
    // 2 and 3 of B's, and the rows / columns of C its 64 x 64 result covers.
    // A symmetric product's A and B stages of one 64-row panel are equal, so
    // a slot serves either operand.  The band of a symmetric product with T
    // tiles of 128 per side is its 3T units of 64 x 64 on and next to the
    // diagonal -- (2t, 2t), (2t, 2t + 1), (2t + 1, 2t + 1) for each t, whose
    // upper triangles cover those of the diagonal tiles -- in groups of four
    // consecutive units, which lie in the panels of tiles t0 and t0 + 1.  A
    // wave past the band's end computes on slot 0 and stores nothing.
    int ua = wm, ub = 2 + wn, rbase = i0 + 64 * wm, cbase = j0 + 64 * wn;
    if constexpr (F32S || XF) {
        if (band) {
            const int u = 4 * q + w, tu = u / 3, v = u - 3 * tu;
            const int pa = 2 * tu + (v == 2), pb = 2 * tu + (v != 0);
            ua = pa - 2 * t0;
            ub = pb - 2 * t0;
            rbase = 64 * pa;
            cbase = 64 * pb;
            if (u >= 3 * tk.tiles_n) {
                ua = ub = 0;
                rbase = tk.M;
            }
        }
    }
    // A mirrored symmetric product is stored bitwise symmetric: on a diagonal
    // tile the lower-left wave stores nothing (rows from M on are masked) and
    // the upper-right one also writes its transpose, as off-diagonal tiles
    // do; a wave on the diagonal stores its upper triangle and mirrors it
    // (below).  (Products that are symmetric only in exact arithmetic, X T'
    // and T'^p M, would otherwise leave the two triangles a rounding apart,
    // and a band unit may read either one as its operand.)
    if (!band && ti == tj && ((tk.trans >> 4) & 1) && ((tk.trans >> 5) & 1) && wm == 1 && wn == 0)
        rbase = tk.M;
    WaveTile<T> wt;
    wt.zero();

    StageLoader<S, TA> la;
    StageLoader<S, TB> lb;
    // in a persistent launch the thread index goes through an opaque copy:
    // values derived from it are then formed per tile, not hoisted out of
    // the tile loop (kept live across it they spilled)
    int tid = threadIdx.x;
    if constexpr (PERSIST) asm volatile("" : "+v"(tid));
    la.t = tid;
    lb.t = tid;
    // A split-K part sums k in [kb, K).  fp32: the operands are offset to
    // k = kb and the loop runs from 0 (a Newton operand's diagonal is found
    // with offset kb); fp64: the loop runs from kb.  The two forms compute the
    // same; each keeps its kernel at the register count of the unsplit loop
    // (measured: the other form costs fp32 an occupancy step, fp64 spills).
    constexpr bool kofs = sizeof(T) == 4;
    const int kb = tk.kb;
    const int kfirst = kofs ? 0 : kb, Kp = kofs ? tk.K - kb : tk.K, dk = kofs ? kb : 0;
    if (kofs) {
        A += a_kc ? (int64_t)kb : (int64_t)kb * tk.lda;
        B += b_kc ? (int64_t)kb : (int64_t)kb * tk.ldb;
    }
    // where C's rows and columns of the wave's result start, less the offsets
    // the accumulator places add (64 wm, 64 wn)
    const int ci0 = rbase - 64 * wm, cj0 = cbase - 64 * wn;
    const S* Ap = (ua < 2 ? As : Bs) + 64 * (ua & 1);
    const S* Bp = (ub < 2 ? As : Bs) + 64 * (ub & 1);
    constexpr bool axpby = AXPBY;   // the launcher picks it from args.epi
    // C <- alpha op(A) op(B) + beta C (the statistics): the old values of C
    // are read in halves of the wave's result, the first half while the last
    // stage's products run (that stage is peeled off the loop, so the stage
    // registers are dead by then and the loaded values need no registers of
    // their own inside the loop), the second half after the first is stored:
    // one exposed round trip per tile instead of one per group of 16
    constexpr int NV = WaveTile<T>::NV, HALF = NV / 2;
    T old[HALF];
    auto load_old = [&](int h0) {
#pragma unroll
        for (int e = 0; e < HALF; ++e) {
            int r, c;
            (void)wt.get(h0 + e, wm, wn, r, c);
            const int i = ci0 + r, j = cj0 + c;
            old[e] = (i < tk.M && j < tk.N) ? C[(int64_t)i * tk.ldc + j] : T(0);
        }
    };
    la.load(A, tk.lda, a_kc, i0, kfirst, tk.M, Kp, a_al, xa, c1, c2, dk);
    lb.load(B, tk.ldb, b_kc, j0, kfirst, tk.N, Kp, b_al, xb, c1, c2, dk);
    if constexpr (axpby) {
        if (Kp > kfirst) {
            int k0 = kfirst;
            for (; k0 + BK < Kp; k0 += BK) {   // every stage but the last
                __syncthreads();
                la.store(As, a_kc);
                lb.store(Bs, b_kc);
                __syncthreads();
                la.load(A, tk.lda, a_kc, i0, k0 + BK, tk.M, Kp, a_al, xa, c1, c2, dk);
                lb.load(B, tk.ldb, b_kc, j0, k0 + BK, tk.N, Kp, b_al, xb, c1, c2, dk);
                if constexpr (F32S) wt.compute_f32(Ap, Bp);
                else wt.compute(Ap, Bp);
            }
            __syncthreads();
            la.store(As, a_kc);
            lb.store(Bs, b_kc);
            __syncthreads();
            load_old(0);
            if constexpr (F32S) wt.compute_f32(Ap, Bp);
            else wt.compute(Ap, Bp);
        } else {
            load_old(0);
        }
    } else {
        for (int k0 = kfirst; k0 < Kp; k0 += BK) {
            __syncthreads();
            la.store(As, a_kc);
            lb.store(Bs, b_kc);
            __syncthreads();
            if (k0 + BK < tk.K) {
                la.load(A, tk.lda, a_kc, i0, k0 + BK, tk.M, Kp, a_al, xa, c1, c2, dk);
                lb.load(B, tk.ldb, b_kc, j0, k0 + BK, tk.N, Kp, b_al, xb, c1, c2, dk);
            }
            if constexpr (F32S) wt.compute_f32(Ap, Bp);
            else wt.compute(Ap, Bp);
        }
    }

    const T alpha = T(args.alpha), beta = T(args.beta);
    // symmetric result computed on upper tiles only: a wave whose part lies
    // off the diagonal also writes its transpose
    const bool mirror = ((tk.trans >> 5) & 1) && rbase != cbase;
    // ... and one on the diagonal forms j >= i only, each value also stored at
    // its transpose (as the split-K sum does)
    const bool sdiag = ((tk.trans >> 4) & 1) && ((tk.trans >> 5) & 1) && rbase == cbase;
    // fp32 results of a wave whose 64 x 64 part is wholly in range mirror
    // with 16-byte stores after its own stores (aligned: ldc and the offsets
    // of such products are multiples of 4)
    const bool vmirror = sizeof(T) == 4 && !AXPBY && mirror && rbase + 64 <= tk.M && cbase + 64 <= tk.N &&
                         (tk.ldc & 3) == 0 && (reinterpret_cast<uintptr_t>(C) & 15) == 0;
    // mirrored values land in the transposed tile, which no workgroup reads
    double nrm = 0.0;
#pragma unroll
    for (int h0 = 0; h0 < NV; h0 += HALF) {
        if constexpr (axpby) {
            if (h0 > 0) load_old(h0);   // (a store may alias it as far as the compiler knows)
        }
#pragma unroll
        for (int e = 0; e < HALF; ++e) {
            int r, c;
            const T v = wt.get(h0 + e, wm, wn, r, c);
            const int i = ci0 + r, j = cj0 + c;
            if (i < tk.M && j < tk.N && (!sdiag || j >= i)) {
                T o = alpha * v;
                if constexpr (axpby) o += beta * old[e];
                C[(int64_t)i * tk.ldc + j] = o;
                if ((mirror && !vmirror) || (sdiag && j > i)) C[(int64_t)j * tk.ldc + i] = o;
                nrm += double(o) * double(o);
            }
        }
    }
    if constexpr (sizeof(T) == 4 && !AXPBY) {
        if (vmirror) wt.store_transposed(C + (int64_t)cj0 * tk.ldc + ci0, tk.ldc, wm, wn, alpha);
    }
    if (tk.norm_slot >= 0 && args.norms) {
        const double s = block_sum_256(nrm, red);
        if (threadIdx.x == 0) args.norms[tk.norm_slot + tr.tile] = s;
    }
    return true;
}

// ROLE only names the instantiation (0: Newton products and statistics, 1 and
// 2: the first and second product of the two-sided apply), so that kernel
// traces and counters tell the launch families apart.
template <typename T, typename TA, typename TB, int MINW, bool AXPBY, bool PERSIST, int ROLE = 0>
__global__ __launch_bounds__(256, MINW) void k_gemm(const GemmTask* __restrict__ tasks,
                                             const TileRef* __restrict__ tiles,
                                             const uint64_t* __restrict__ bases, GemmArgs args) {
    using S = typename std::conditional<kStageF32<T, TA, TB>, float, T>::type;
    // only the Newton products take the operand transform
    constexpr bool XF = ROLE == 0 && !kStageF32<T, TA, TB>;
    constexpr int BK = GemmTraits<S>::BK;
    constexpr int P = BM + GemmTraits<S>::PADE;
    __shared__ __align__(16) S As[BK * P];
    __shared__ __align__(16) S Bs[BK * P];
    __shared__ double red[4];
    if constexpr (PERSIST) {
        // the table is sorted by gating id and the live ids are a prefix, so
        // the first gated tile a workgroup meets ends it; a group of `chain`
        // products runs in order on one workgroup (the barrier between them
        // also makes each product's stores visible to the next one's loads)
        const int C = args.chain > 1 ? args.chain : 1;
        bool first = true;
        for (int e0 = blockIdx.x * C; e0 < args.ntiles; e0 += gridDim.x * C) {
            bool live = true;
            for (int j = 0; j < C && e0 + j < args.ntiles; ++j) {
                if (!first) __syncthreads();   // the previous tile's LDS reads and stores are done
                first = false;
                if (!gemm_tile<T, TA, TB, AXPBY, XF, PERSIST>(e0 + j, tasks, tiles, bases, args, As, Bs, red)) {
                    live = false;
                    break;
                }
            }
            if (!live) break;
        }
    } else {
        (void)gemm_tile<T, TA, TB, AXPBY, XF, PERSIST>(blockIdx.x, tasks, tiles, bases, args, As, Bs, red);
    }
}

// ================================== split-precision (bf16x3) products
// C = A B^T with fp32 A (M x K) and B (N x K), both rows k-contiguous, on the
// bf16 matrix cores (v_mfma_f32_32x32x16_bf16): every operand x is split
// into hi = bf16(x) and lo = bf16(x - hi) as it is staged into LDS, and C
// accumulates lo*hi + hi*lo + hi*hi in fp32.  The dropped lo*lo term and the
// rounding of lo leave about 2^-16 of |a||b| per term (fp32 products: 2^-24),
// well inside the apply's update bar; the products run at the bf16 rate.
// 128 x 128 tiles, four waves of 64 x 64 (2 x 2 tiles of 32 x 32), BK = 32
// per LDS stage with the next stage prefetched into registers.  The operand
// of lane l in one instruction is row l % 32 and k in [8 (l / 32), +8) of
// the 16-deep step, the same for A and B (any k order shared by both gives
// the same sums; checked on the device), read as one 16-byte LDS load; the
// row pitch of 40 bf16 (80 bytes) puts the rows of eight lanes on distinct
// banks.  ADAG: the tiles also take B's elements (a gradient block) through
// the Adagrad accumulator a <- a + g^2 and sum (g / (sqrt(a) + delta))^2 for
// the graft, each element of B once per launch: the k-stages of a row of B
// are spread over the tiles that read it.
constexpr int kNtBK = 32;
constexpr int kNtP = kNtBK + 8;

typedef __bf16 nt_bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 nt_bf16x4 __attribute__((ext_vector_type(4)));
typedef float nt_acc_t __attribute__((ext_vector_type(16)));

// Rows [r0, r0 + 128) x k [k0, k0 + 32) of a k-contiguous fp32 matrix into
// registers: thread t takes rows r0 + t/8 + 32p (p < 4), k = k0 + 4 (t % 8) + e.
// Out-of-range elements are zero.  UNIFORM: a stage wholly in range takes a
// path without per-lane checks (measured: faster in the product with the
// Adagrad pass, slower in the other, whose registers it raises).
template <bool UNIFORM>
__device__ __forceinline__ void nt_load(const float* __restrict__ X, int ld, int r0, int R, int k0,
                                        int K, bool aligned, float4 (&v)[4]) {
    const int t = threadIdx.x, kq = t & 7, rr = t >> 3;
    const int k = k0 + 4 * kq;
    const bool kin = aligned && k0 + kNtBK <= K;
    if (UNIFORM && kin && r0 + 128 <= R) {
#pragma unroll
        for (int p = 0; p < 4; ++p)
            v[p] = *reinterpret_cast<const float4*>(X + (int64_t)(r0 + rr + 32 * p) * ld + k);
        return;
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int r = r0 + rr + 32 * p;
        if (kin && r < R) {
            v[p] = *reinterpret_cast<const float4*>(X + (int64_t)r * ld + k);
        } else {
            float x[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = (r < R && k + e < K) ? X[(int64_t)r * ld + k + e] : 0.f;
            v[p] = make_float4(x[0], x[1], x[2], x[3]);
        }
    }
}

// Splits the thread's 16 values into hi / lo bf16 and stores them at rows
// t/8 + 32p, k 4 (t % 8) .. +3 of the stage.
__device__ __forceinline__ void nt_store(const float4 (&v)[4], __bf16* H, __bf16* L) {
    const int t = threadIdx.x, kq = t & 7, rr = t >> 3;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const float x[4] = {v[p].x, v[p].y, v[p].z, v[p].w};
        nt_bf16x4 h, l;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            h[e] = (__bf16)x[e];
            l[e] = (__bf16)(x[e] - (float)h[e]);
        }
        const int o = (rr + 32 * p) * kNtP + 4 * kq;
        *reinterpret_cast<nt_bf16x4*>(H + o) = h;
        *reinterpret_cast<nt_bf16x4*>(L + o) = l;
    }
}

template <bool ADAG>
__global__ __launch_bounds__(256, ADAG ? 2 : 3) void k_gemm_nt3(const NtTask* __restrict__ tasks,
                                                    const TileRef* __restrict__ tiles,
                                                    const uint64_t* __restrict__ bases, NtArgs args) {
    __shared__ __align__(16) __bf16 Ah[BM * kNtP];
    __shared__ __align__(16) __bf16 Al[BM * kNtP];
    __shared__ __align__(16) __bf16 Bh[BN * kNtP];
    __shared__ __align__(16) __bf16 Bl[BN * kNtP];
    __shared__ double red[4];
    const TileRef tr = tiles[blockIdx.x];
    const NtTask tk = tasks[tr.task];
    const int ti = tr.tile / tk.tiles_n, tj = tr.tile % tk.tiles_n;
    const int i0 = ti * BM, j0 = tj * BN;
    const float* A = base_ptr<const float>(bases, tk.a_base, tk.a_off);
    const float* B = base_ptr<const float>(bases, tk.b_base, tk.b_off);
    float* C = base_ptr<float>(bases, tk.c_base, tk.c_off);
    const bool a_al = ((reinterpret_cast<uintptr_t>(A) & 15) == 0) && (tk.lda % 4 == 0);
    const bool b_al = ((reinterpret_cast<uintptr_t>(B) & 15) == 0) && (tk.ldb % 4 == 0);
    // the Adagrad pass over B's elements, spread over the tile rows: tile
    // (ti, tj) takes the k-stages s with s mod (tile rows) == ti of B's rows
    // [128 tj, +128), so each element is taken once (uniform per workgroup)
    const bool adag = ADAG && tk.acc_off >= 0;
    const int tiles_m = (tk.M + BM - 1) / BM;
    auto mine = [&](int k0) { return adag && (k0 / kNtBK) % tiles_m == ti; };
    float* acc = args.arena + (adag ? tk.acc_off : 0);
    const bool c_al = b_al && ((reinterpret_cast<uintptr_t>(acc) & 15) == 0);
    const float delta = args.delta;
    double asum = 0.0;

    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int wm = w >> 1, wn = w & 1, h = lane >> 5, c = lane & 31;
    nt_acc_t cc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) cc[i][j][v] = 0.f;

    float4 av[4], bv[4], gv[4];
    auto acc_load = [&](int k0) {
        const int kq = t & 7, rr = t >> 3, k = k0 + 4 * kq;
        const bool kin = c_al && k0 + kNtBK <= tk.K;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int r = j0 + rr + 32 * p;
            if (kin && r < tk.N) {
                gv[p] = *reinterpret_cast<const float4*>(acc + (int64_t)r * tk.ldb + k);
            } else {
                float x[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    x[e] = (r < tk.N && k + e < tk.K) ? acc[(int64_t)r * tk.ldb + k + e] : 0.f;
                gv[p] = make_float4(x[0], x[1], x[2], x[3]);
            }
        }
    };
    // a <- a + g^2 on the stage's elements of B, and their share of ||A||^2
    auto acc_update = [&](int k0) {
        const int kq = t & 7, rr = t >> 3, k = k0 + 4 * kq;
        const bool kin = c_al && k0 + kNtBK <= tk.K;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int r = j0 + rr + 32 * p;
            const float g[4] = {bv[p].x, bv[p].y, bv[p].z, bv[p].w};
            float a[4] = {gv[p].x, gv[p].y, gv[p].z, gv[p].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                a[e] += g[e] * g[e];
                const float Ae = g[e] / (sqrtf(a[e]) + delta);
                if (r < tk.N && k + e < tk.K) asum += (double)(Ae * Ae);
            }
            if (kin && r < tk.N) {
                *reinterpret_cast<float4*>(acc + (int64_t)r * tk.ldb + k) = make_float4(a[0], a[1], a[2], a[3]);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (r < tk.N && k + e < tk.K) acc[(int64_t)r * tk.ldb + k + e] = a[e];
            }
        }
    };

    nt_load<ADAG>(A, tk.lda, i0, tk.M, 0, tk.K, a_al, av);
    nt_load<ADAG>(B, tk.ldb, j0, tk.N, 0, tk.K, b_al, bv);
    if (mine(0)) acc_load(0);
    for (int k0 = 0; k0 < tk.K; k0 += kNtBK) {
        if (mine(k0)) acc_update(k0);
        __syncthreads();   // the previous stage's LDS reads are done
        nt_store(av, Ah, Al);
        nt_store(bv, Bh, Bl);
        __syncthreads();
        if (k0 + kNtBK < tk.K) {
            nt_load<ADAG>(A, tk.lda, i0, tk.M, k0 + kNtBK, tk.K, a_al, av);
            nt_load<ADAG>(B, tk.ldb, j0, tk.N, k0 + kNtBK, tk.K, b_al, bv);
            if (mine(k0 + kNtBK)) acc_load(k0 + kNtBK);
        }
#pragma unroll
        for (int kk = 0; kk < kNtBK; kk += 16) {
            nt_bf16x8 ah[2], al[2], bh[2], bl[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int o = (wm * 64 + i * 32 + c) * kNtP + kk + 8 * h;
                ah[i] = *reinterpret_cast<const nt_bf16x8*>(Ah + o);
                al[i] = *reinterpret_cast<const nt_bf16x8*>(Al + o);
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int o = (wn * 64 + j * 32 + c) * kNtP + kk + 8 * h;
                bh[j] = *reinterpret_cast<const nt_bf16x8*>(Bh + o);
                bl[j] = *reinterpret_cast<const nt_bf16x8*>(Bl + o);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    cc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[i], bh[j], cc[i][j], 0, 0, 0);
                    cc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[i], bl[j], cc[i][j], 0, 0, 0);
                    cc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[i], bh[j], cc[i][j], 0, 0, 0);
                }
        }
    }

    // C and the tile's ||C||^2 (lane (h, c), register v: row 8 (v/4) + 4h + v%4, column c)
    double nrm = 0.0;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int r = i0 + wm * 64 + i * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
                const int col = j0 + wn * 64 + j * 32 + c;
                if (r < tk.M && col < tk.N) {
                    const float o = cc[i][j][v];
                    C[(int64_t)r * tk.ldc + col] = o;
                    nrm += double(o) * double(o);
                }
            }
    if (tk.norm_slot >= 0 && args.norms) {
        const double sn = block_sum_256(nrm, red);
        if (t == 0) args.norms[tk.norm_slot + tr.tile] = sn;
    }
    if (adag) {
        const double sa = block_sum_256(asum, red);
        if (t == 0) args.partA[tk.acc_slot + ti * tk.tiles_n + tj] = sa;
    }
}

// ====================================================== statistics <= 128
// L <- beta L + alpha G G^T and R <- beta R + alpha G^T G for one block of at
// most 128 x 128 per workgroup: G is read from HBM once into LDS (fp32,
// zero-padded to 128 x 128) and both products run on fp64 MFMA
// (v_mfma_f64_16x16x4f64) from that copy; fp32 x fp32 products are exact in
// fp64.  L and R are symmetric, so only their upper triangles are formed and
// stored: wave 0 takes the two diagonal 64 x 64 quadrants of L (10 of 16
// 16x16 tiles each), wave 1 the off-diagonal quadrant of L, waves 2 and 3 the
// same for R.  The lower triangle of the stored matrix is not maintained.
constexpr int kGP = 132;  // LDS row pitch (floats): 16-byte aligned rows

typedef double gd4 __attribute__((ext_vector_type(4)));
typedef float gf4 __attribute__((ext_vector_type(4)));

// One 64 x 64 quadrant (qi, qj) of L = G G^T (RSIDE = false) or R = G^T G.
// DIAG: qi == qj, only tiles i <= j are formed.  Lane group g supplies
// k = k0 + 4g + s in MFMA step s.
template <bool DIAG, bool RSIDE, int JLO = 0, int JHI = 4>
__device__ __forceinline__ void gram_quadrant(const float* Gs, int qi, int qj, int K, double* S,
                                              int ldS, int nvalid, double alpha, double beta,
                                              int c, int g) {
    if (qi * 64 >= nvalid || qj * 64 + JLO * 16 >= nvalid) return;
    gd4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = gd4{0.0, 0.0, 0.0, 0.0};
    for (int k0 = 0; k0 < K; k0 += 16) {
        if (!RSIDE) {
            gf4 a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                a[i] = *reinterpret_cast<const gf4*>(&Gs[(qi * 64 + i * 16 + c) * kGP + k0 + 4 * g]);
#pragma unroll
            for (int j = JLO; j < JHI; ++j)
                b[j] = DIAG ? a[j]
                            : *reinterpret_cast<const gf4*>(&Gs[(qj * 64 + j * 16 + c) * kGP + k0 + 4 * g]);
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = JLO; j < JHI; ++j)
                        if (!DIAG || i <= j)
                            acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(
                                (double)a[i][s], (double)b[j][s], acc[i][j], 0, 0, 0);
        } else {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const float* row = &Gs[(k0 + 4 * g + s) * kGP];
                double a[4], b[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) a[i] = (double)row[qi * 64 + i * 16 + c];
#pragma unroll
                for (int j = JLO; j < JHI; ++j) b[j] = DIAG ? a[j] : (double)row[qj * 64 + j * 16 + c];
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = JLO; j < JHI; ++j)
                        if (!DIAG || i <= j)
                            acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], b[j], acc[i][j], 0, 0, 0);
            }
        }
    }
    // read-modify-write of the statistics, two tiles at a time: their eight
    // loads in flight before the first store (the stores could alias later
    // loads as far as the compiler knows, so it would not hoist them)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j0 = JLO; j0 < JHI; j0 += 2) {
            double old[2][4];
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const int j = j0 + jj;
                if (j >= JHI || (DIAG && i > j)) continue;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int r = qi * 64 + i * 16 + g + 4 * v, q = qj * 64 + j * 16 + c;
                    old[jj][v] = (r < nvalid && q < nvalid) ? S[(int64_t)r * ldS + q] : 0.0;
                }
            }
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const int j = j0 + jj;
                if (j >= JHI || (DIAG && i > j)) continue;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int r = qi * 64 + i * 16 + g + 4 * v, q = qj * 64 + j * 16 + c;
                    if (r < nvalid && q < nvalid)
                        S[(int64_t)r * ldS + q] = alpha * acc[i][j][v] + beta * old[jj][v];
                }
            }
        }
}

// The statistics of one block of at most 128 x 128 on a 512-thread
// workgroup; Gs: 128 x kGP floats of LDS.
__device__ __forceinline__ void gram128_block(const GramJob& job, const uint64_t* __restrict__ bases,
                                              double* __restrict__ stats, double alpha, double beta,
                                              float* Gs) {
    const GramJob jb = job;
    const float* G = base_ptr<const float>(bases, jb.g_base, jb.g_off);
    const int t = threadIdx.x;
    const int mb = jb.mb, nb = jb.nb, ld = jb.ldg;

    // ---- stage G (rows x cols) into LDS, zero padded
    const bool vec = (nb % 4 == 0) && (ld % 4 == 0) && ((reinterpret_cast<uintptr_t>(G) & 15) == 0);
    {
        const int c4 = t & 31, r0 = t >> 5;   // 32 float4 per row, 16 rows per pass
        float4 buf[8];
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            const int r = r0 + 16 * p, c = 4 * c4;
            if (r < mb && c < nb) {
                if (vec) {
                    buf[p] = *reinterpret_cast<const float4*>(G + (int64_t)r * ld + c);
                } else {
                    buf[p].x = G[(int64_t)r * ld + c];
                    buf[p].y = (c + 1 < nb) ? G[(int64_t)r * ld + c + 1] : 0.f;
                    buf[p].z = (c + 2 < nb) ? G[(int64_t)r * ld + c + 2] : 0.f;
                    buf[p].w = (c + 3 < nb) ? G[(int64_t)r * ld + c + 3] : 0.f;
                }
            } else {
                buf[p] = make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
#pragma unroll
        for (int p = 0; p < 8; ++p)
            *reinterpret_cast<float4*>(&Gs[(r0 + 16 * p) * kGP + 4 * c4]) = buf[p];
    }
    __syncthreads();

    // eight waves: L and R each as two diagonal quadrants (10 tiles each) and
    // the off-diagonal quadrant split into two halves of 8 tiles
    const int lane = t & 63, w = t >> 6;
    const int c = lane & 15, g = lane >> 4;
    const int KL = (nb + 15) & ~15, KR = (mb + 15) & ~15;
    double* L = stats + jb.l_off;
    double* R = stats + jb.r_off;
    switch (w) {
        case 0: gram_quadrant<true, false>(Gs, 0, 0, KL, L, jb.ld_l, mb, alpha, beta, c, g); break;
        case 1: gram_quadrant<true, false>(Gs, 1, 1, KL, L, jb.ld_l, mb, alpha, beta, c, g); break;
        case 2: gram_quadrant<false, false, 0, 2>(Gs, 0, 1, KL, L, jb.ld_l, mb, alpha, beta, c, g); break;
        case 3: gram_quadrant<false, false, 2, 4>(Gs, 0, 1, KL, L, jb.ld_l, mb, alpha, beta, c, g); break;
        case 4: gram_quadrant<true, true>(Gs, 0, 0, KR, R, jb.ld_r, nb, alpha, beta, c, g); break;
        case 5: gram_quadrant<true, true>(Gs, 1, 1, KR, R, jb.ld_r, nb, alpha, beta, c, g); break;
        case 6: gram_quadrant<false, true, 0, 2>(Gs, 0, 1, KR, R, jb.ld_r, nb, alpha, beta, c, g); break;
        default: gram_quadrant<false, true, 2, 4>(Gs, 0, 1, KR, R, jb.ld_r, nb, alpha, beta, c, g); break;
    }
}

__global__ __launch_bounds__(512, 4) void k_gram128(const GramJob* __restrict__ jobs,
                                                   const uint64_t* __restrict__ bases,
                                                   double* __restrict__ stats, double alpha,
                                                   double beta) {
    __shared__ __align__(16) float Gs[128 * kGP];
    gram128_block(jobs[blockIdx.x], bases, stats, alpha, beta, Gs);
}

// ================================================================ Lanczos
// Extreme Ritz values of a symmetric matrix from `steps` Lanczos steps (no
// reorthogonalisation: lost orthogonality only duplicates converged extreme
// values, it never moves the largest Ritz value above lambda_max).  Vectors
// in fp64 in LDS; the matrix is read in fp32 column-wise (coalesced; the
// matrix is symmetric so S v = S^T v).  The tridiagonal's extremes come from
// Sturm-count multisection.
constexpr int kLanczosMaxN = 1024;
constexpr int kLanczosMaxSteps = 64;

// One step of the Sturm recurrence d_k = (a_k - x) - b_{k-1}^2 / d_{k-1}, the
// quotient taken as b^2 times the hardware reciprocal refined by one Newton
// step (full double accuracy; the raw reciprocal is kept when d_{k-1} is
// infinite, where the refinement would give NaN and the quotient is 0).
__device__ __forceinline__ double sturm_step(double d, double a_minus_x, double b2) {
    double r = __builtin_amdgcn_rcp(d);
    const double rr = fma(r, fma(-d, r, 1.0), r);
    r = rr == rr ? rr : r;
    d = fma(-b2, r, a_minus_x);
    return d == 0.0 ? -1e-300 : d;
}

// Largest eigenvalue of the m x m tridiagonal (al, be) by Sturm-count
// multisection on one wave: every lane counts the eigenvalues below two
// points of the bracket (two independent recurrences in flight), so each
// round shrinks it 129-fold, until the bracket is within rtol of its upper
// end (which is returned).  NaN for non-finite input.
__device__ __forceinline__ double tridiag_max_wave(const double* al, const double* be, int m,
                                                   double rtol = 1e-15) {
    const int lane = threadIdx.x & 63;
    double lo = 0.0, hi = 0.0;
    bool finite = true;
    for (int k = 0; k < m; ++k) {
        const double r = (k ? fabs(be[k - 1]) : 0.0) + (k + 1 < m ? fabs(be[k]) : 0.0);
        if (!isfinite(al[k]) || !isfinite(r)) finite = false;
        lo = k ? fmin(lo, al[k] - r) : al[k] - r;
        hi = k ? fmax(hi, al[k] + r) : al[k] + r;
    }
    if (!finite) return NAN;
    for (int round = 0; round < 12; ++round) {
        if (!(hi - lo > rtol * fmax(fabs(lo), fabs(hi)))) break;
        const double h = (hi - lo) / 129.0;
        const double x0 = lo + h * (double)(2 * lane + 1), x1 = lo + h * (double)(2 * lane + 2);
        double d0 = al[0] - x0, d1 = al[0] - x1;
        if (d0 == 0.0) d0 = -1e-300;
        if (d1 == 0.0) d1 = -1e-300;
        int c0 = d0 < 0.0, c1 = d1 < 0.0;
        for (int k = 1; k < m; ++k) {
            const double b2 = be[k - 1] * be[k - 1], a = al[k];
            d0 = sturm_step(d0, a - x0, b2);
            d1 = sturm_step(d1, a - x1, b2);
            c0 += d0 < 0.0;
            c1 += d1 < 0.0;
        }
        // the first point above every eigenvalue (point j = 2 lane + 1 + s)
        const uint64_t m0 = __ballot(c0 >= m), m1 = __ballot(c1 >= m);
        int j = 129;
        if (m0) j = 2 * (__ffsll((unsigned long long)m0) - 1) + 1;
        if (m1) j = min(j, 2 * (__ffsll((unsigned long long)m1) - 1) + 2);
        if (j == 129) {
            lo = lo + h * 128.0;
        } else {
            const double nlo = lo + h * (double)(j - 1), nhi = lo + h * (double)j;
            lo = nlo;
            hi = nhi;
        }
    }
    return hi;
}

// Residual norm beta_m |y_m| of the top Ritz pair (theta, y) of the m x m
// Lanczos tridiagonal (al, be; be[m-1] couples it to the next Lanczos
// vector): some eigenvalue of the matrix lies within it of theta.  y_m comes
// from one step of inverse iteration with the shift sigma just above theta,
// started from e_m: with T - sigma I = L D L^T (negative definite, so the
// pivots d_j are the Sturm recurrence and never vanish), x = (T - sigma I)^-1
// e_m has x_m = 1/d_m and x_j = -l_j x_{j+1} (l_j = be_j / d_j), so
// y_m^2 = x_m^2 / |x|^2 = 1 / S with S = sum_j prod_{i >= j} l_i^2, formed
// forward as S <- S l_j^2 + 1.  No arrays; an overflow of S means a
// converged pair (residual 0).
__device__ __forceinline__ double ritz_residual(const double* al, const double* be, int m,
                                                double theta) {
    const double sigma = theta + 1e-10 * fabs(theta);
    double d = al[0] - sigma, S = 1.0;
    for (int j = 0; j + 1 < m; ++j) {
        const double b2 = be[j] * be[j];
        S = fma(S, b2 / (d * d), 1.0);
        d = (al[j + 1] - sigma) - b2 / d;
    }
    return fabs(be[m - 1]) / sqrt(S);
}

// The adaptive stop's test on one wave: is the top Ritz pair of the m x m
// tridiagonal within tol of converged?  Out of line, so that the registers
// of the multisection are not added to those of the kernels that inline the
// Lanczos loop (the fused root).
__device__ __attribute__((noinline)) bool ritz_converged(const double* al, const double* be, int m,
                                                        double tol) {
    const double th = tridiag_max_wave(al, be, m);
    return !(ritz_residual(al, be, m, th) > tol * th);
}

// Check points of the adaptive Lanczos stop: after 12 steps, every 4th step
// up to 32 and every 8th after (a top Ritz pair's residual falls steadily
// until it is converged; sparse checks keep the multisection's cost small).
__device__ __forceinline__ bool lanczos_check_step(int m) {
    return m >= 12 && ((m <= 32 && (m & 3) == 0) || (m & 7) == 0);
}


// 128 x 128 fp32 matrices in LDS ("slots"): row pitch 129 floats, the column
// index stored with its bits 2 and 5 exchanged.  With this layout the MFMA
// operand reads of the fused kernels (lane (h, c) at row c, column k + 4h, or
// at row k + 4h, column c), their strip stores and the row reads of the
// Lanczos product each hit 64 distinct banks, and every address is a
// per-lane base plus a compile-time offset.
constexpr int kSP = 129;
__host__ __device__ constexpr int pcol(int j) { return (j & ~0x24) | ((j & 4) << 3) | ((j >> 3) & 4); }
__device__ __forceinline__ int sidx(int r, int j) { return r * kSP + pcol(j); }

// Stages the symmetric n x n matrix whose upper triangle is at S (row pitch
// ld, n <= 128) into a slot in fp32, zero outside n x n: sixteen loads in
// flight per thread, then their stores (each upper element and its mirror).
template <typename TM>
__device__ __forceinline__ void stage_sym(float* slot, const TM* S, int n, int ld) {
    constexpr int kB = 16;
    for (int e0 = 0; e0 < 128 * 128; e0 += 256 * kB) {
        float x[kB];
#pragma unroll
        for (int u = 0; u < kB; ++u) {
            const int e = e0 + 256 * u + threadIdx.x, i = e >> 7, j = e & 127;
            x[u] = (j >= i && j < n) ? (float)S[(int64_t)i * ld + j] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < kB; ++u) {
            const int e = e0 + 256 * u + threadIdx.x, i = e >> 7, j = e & 127;
            if (j >= i) {
                slot[sidx(i, j)] = x[u];
                slot[sidx(j, i)] = x[u];
            }
        }
    }
}

// Scratch of the slot Lanczos.
struct LanczosSlot {
    alignas(16) float vf[128];   // v rounded to fp32, the operand of the product
    double al[kLanczosMaxSteps], be[kLanczosMaxSteps];
    double ra[4], rb[4];
    double res;
    int stop;
};

// Largest Ritz value of the symmetric n x n matrix held in a slot (entries
// outside n x n zero, or an identity block that is decoupled from the rest)
// after up to `steps` Lanczos steps.  Thread (wave w, lane l) owns row
// r = 32w + l%32 and half of its columns; the two halves meet in one shuffle,
// so v_r, the previous v_r and the new w_r stay in registers and only v is
// shared through LDS.  The product S v is formed in fp32 (the slot holds S in
// fp32; v rounded to fp32, read four entries at a time as an LDS broadcast;
// eight fp32 partial sums of eight terms each), which perturbs the Ritz
// values by about 1e-6 of lambda_max; the recurrence itself runs in fp64.
// ROWREG: the thread's 64 matrix entries are read into registers once.
// Sums run in a fixed order: every thread sees the same alpha and beta, so
// the early stop is uniform.  tol > 0: stop at the first check point where
// the top Ritz pair's residual is at most tol theta (theta is then within
// tol theta of an eigenvalue, the largest one for a start vector that meets
// its eigenvector), at most `steps` steps.
template <bool ROWREG>
__device__ __forceinline__ double lanczos_slot(const float* slot, int n, int steps, LanczosSlot& L,
                                               double tol = 0.0) {
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int r = 32 * w + (lane & 31), hf = lane >> 5;
    steps = min(steps, min(n, kLanczosMaxSteps));
    double v = 0.0;
    if (r < n) {
        uint32_t hsh = (uint32_t)r * 2654435761u + 0x9E3779B9u;
        hsh ^= hsh >> 15; hsh *= 2246822519u; hsh ^= hsh >> 13;
        v = 0.5 + (double)(hsh & 0xFFFFFF) / 16777216.0;
    }
    {
        const double s2 = wave_sum(hf == 0 ? v * v : 0.0);
        if (lane == 0) L.ra[w] = s2;
        __syncthreads();
        v /= sqrt((L.ra[0] + L.ra[1]) + (L.ra[2] + L.ra[3]));
    }
    if (hf == 0) L.vf[r] = (float)v;
    if (t == 0) L.stop = 0;
    // physical columns 32hf + 64u + q hold logical columns pcol(64u + q) + 4hf;
    // pcol keeps bits 0-1, so four consecutive q are four consecutive columns
    const float* Ar = slot + r * kSP + 32 * hf;
    const float* vb = L.vf + 4 * hf;
    float row[ROWREG ? 64 : 1];
    if constexpr (ROWREG) {
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int q = 0; q < 32; ++q) row[32 * u + q] = Ar[64 * u + q];
    }
    __syncthreads();
    double v0 = 0.0, beta_prev = 0.0;
    int m_used = steps;
    for (int k = 0; k < steps; ++k) {
        float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int a = 0; a < 8; ++a) {
                const float4 vv = *reinterpret_cast<const float4*>(vb + pcol(64 * u + 4 * a));
                float x[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = ROWREG ? row[32 * u + 4 * a + e] : Ar[64 * u + 4 * a + e];
                s[4 * u + 0] = fmaf(x[0], vv.x, s[4 * u + 0]);
                s[4 * u + 1] = fmaf(x[1], vv.y, s[4 * u + 1]);
                s[4 * u + 2] = fmaf(x[2], vv.z, s[4 * u + 2]);
                s[4 * u + 3] = fmaf(x[3], vv.w, s[4 * u + 3]);
            }
        double wr = (((double)s[0] + (double)s[1]) + ((double)s[2] + (double)s[3])) +
                    (((double)s[4] + (double)s[5]) + ((double)s[6] + (double)s[7]));
        wr += __shfl_xor(wr, 32, 64);
        const double d = wave_sum(hf == 0 ? wr * v : 0.0);
        if (lane == 0) L.ra[w] = d;
        __syncthreads();
        const double alpha = (L.ra[0] + L.ra[1]) + (L.ra[2] + L.ra[3]);
        const double x = wr - alpha * v - beta_prev * v0;
        const double q2 = wave_sum(hf == 0 ? x * x : 0.0);
        if (lane == 0) L.rb[w] = q2;
        __syncthreads();
        const double beta = sqrt((L.rb[0] + L.rb[1]) + (L.rb[2] + L.rb[3]));
        if (t == 0) {
            L.al[k] = alpha;
            L.be[k] = beta;
        }
        if (!(beta > 1e-13 * fabs(alpha)) || !isfinite(alpha) || !isfinite(beta)) {
            m_used = k + 1;
            break;
        }
        if (tol > 0.0 && k + 1 < steps && lanczos_check_step(k + 1)) {
            __syncthreads();   // al, be of this step written
            if (w == 0) {
                const bool conv = ritz_converged(L.al, L.be, k + 1, tol);
                if (lane == 0) L.stop = conv;
            }
            __syncthreads();
            if (L.stop) {      // uniform: every thread reads the same word
                m_used = k + 1;
                break;
            }
        }
        v0 = v;
        v = x / beta;
        if (hf == 0) L.vf[r] = (float)v;
        beta_prev = beta;
        __syncthreads();
    }
    __syncthreads();   // al, be complete
    if (w == 0) {
        const double lm = tridiag_max_wave(L.al, L.be, m_used);
        if (lane == 0) L.res = lm;
    }
    __syncthreads();
    return L.res;
}

// Writes one factor's Lanczos result: mode 0 (statistics): lambda_max, eps,
// status; mode 1 (root): kappa estimate and, in AUTO mode, the routing flag.
__device__ __forceinline__ void lanczos_finish(const LanczosArgs& args, const LanczosJob& jb,
                                               bool finite, double lmax) {
    FactorDiag& dg = args.diag[jb.factor];
    if (args.mode == 0) {
        // statistics: lambda_max -> eps; status bits for the Newton pass
        int st = 0;
        if (!finite) st |= SHAMPOO_FACTOR_NONFINITE_INPUT_;
        else if (!(lmax > 0.0)) st |= SHAMPOO_FACTOR_ZERO_;
        dg.lambda_max = lmax;
        dg.eps = (st == 0) ? args.eps_rel * lmax : 0.0;
        dg.status = st;
        dg.kappa_est = 0.0;
        dg.residual = 0.0;
        dg.iters = 0;
        if (args.prec) args.prec[jb.factor] = args.route_all_fp64 ? 1 : 0;
    } else {
        // root: lambda_max(P) = (lambda_min(S) + eps)^(-1/p) -> kappa estimate.
        // A factor whose fp32 iteration went non-finite or did not converge is
        // routed to fp64 as well.
        const int bad_in = dg.status & (SHAMPOO_FACTOR_NONFINITE_INPUT_ | SHAMPOO_FACTOR_ZERO_);
        double kap = 0.0;
        if (!bad_in && finite && lmax > 0.0) kap = (dg.lambda_max + dg.eps) * pow(lmax, (double)jb.p);
        dg.kappa_est = kap;
        if (args.prec && args.auto_route) {
            const bool weak = (dg.status & (SHAMPOO_FACTOR_NONFINITE_ROOT_ | SHAMPOO_FACTOR_RESIDUAL_HIGH_)) != 0;
            args.prec[jb.factor] = (!bad_in && (kap > args.threshold || weak)) ? 1 : 0;
        }
    }
}

// Largest eigenvalue estimate of one symmetric factor (n <= 128) per
// workgroup: the matrix (upper triangle) is staged into a slot in fp32 and
// lanczos_slot runs on it.
template <typename TM>
__global__ __launch_bounds__(256, 2) void k_lanczos(const LanczosJob* __restrict__ jobs,
                                                   const TM* __restrict__ arena, LanczosArgs args) {
    __shared__ __align__(16) float slot[128 * kSP];
    __shared__ LanczosSlot lz;
    const LanczosJob jb = jobs[blockIdx.x];
    stage_sym(slot, arena + jb.off, jb.n, jb.ld);
    __syncthreads();
    const double lmax = lanczos_slot<true>(slot, jb.n, args.steps, lz, args.tol);
    if (threadIdx.x == 0) lanczos_finish(args, jb, isfinite(lmax), lmax);
}

// Same for one factor of 129..1024 per workgroup of 1024 threads, matrix read
// from memory, upper triangle only (half the bytes of the full matrix): wave w
// takes rows i = w (mod 16) four at a time, lane l columns l + 64m >= i
// (coalesced row segments) against v held in registers; each row's dot
// product is a fixed-order sum over the wave, and the mirrored entries' terms
// collect per lane and column, then over the sixteen waves in wave order.
// Vectors in fp64 in LDS.
struct LanczosBig {
    double v0[kLanczosMaxN], v1[kLanczosMaxN], wv[kLanczosMaxN];
    double part[16 * kLanczosMaxN];   // per-wave column sums of the product
    double al[kLanczosMaxSteps], be[kLanczosMaxSteps];
    double red[16];
    double res;
    int m_used, stop;
    int rstop;   // the adaptive stop's decision at the last check point
};

__device__ __forceinline__ double block_sum_512(double v, double* red) {
    v = wave_sum(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    return ((red[0] + red[1]) + (red[2] + red[3])) + ((red[4] + red[5]) + (red[6] + red[7]));
}

__device__ __forceinline__ double block_sum_1024(double v, double* red) {
    v = wave_sum(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    double s0 = 0.0, s1 = 0.0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        s0 += red[k];
        s1 += red[8 + k];
    }
    return s0 + s1;
}

template <typename TM, int NM>
__global__ __launch_bounds__(1024) void k_lanczos_big(const LanczosJob* __restrict__ jobs,
                                                    const TM* __restrict__ arena, LanczosArgs args) {
    __shared__ LanczosBig L;
    const LanczosJob jb = jobs[blockIdx.x];
    const int n = jb.n, ld = jb.ld;
    const TM* S = arena + jb.off;
    const int t = threadIdx.x, w = t >> 6, l = t & 63;
    const int steps = min(args.steps, min(n, kLanczosMaxSteps));
    if (n > 64 * NM) {   // not launched so (the host picks NM); a visible failure if it were
        if (t == 0) lanczos_finish(args, jb, false, 0.0);
        return;
    }

    double s2 = 0.0;
    for (int i = t; i < n; i += 1024) {
        uint32_t hsh = (uint32_t)i * 2654435761u + 0x9E3779B9u;
        hsh ^= hsh >> 15; hsh *= 2246822519u; hsh ^= hsh >> 13;
        const double x = 0.5 + (double)(hsh & 0xFFFFFF) / 16777216.0;
        L.v1[i] = x;
        L.v0[i] = 0.0;
        s2 += x * x;
    }
    const double inv = 1.0 / sqrt(block_sum_1024(s2, L.red));
    for (int i = t; i < n; i += 1024) L.v1[i] *= inv;
    if (t == 0) {
        L.m_used = steps;
        L.rstop = 0;
    }
    __syncthreads();

    double beta_prev = 0.0;
    for (int k = 0; k < steps; ++k) {
        // w = S v from the upper triangle of S only (the matrix is symmetric):
        // row i's entries j >= i give its dot product with v (summed over the
        // wave), and each entry j > i also adds S_ij v_i to the lane's
        // partial of w_j.  v in registers; each wave takes rows w, w + 16,
        // ..., with all of a row's loads in flight at once.
        double vr[NM], wc[NM];
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            vr[m] = (l + 64 * m < n) ? L.v1[l + 64 * m] : 0.0;
            wc[m] = 0.0;
        }
        for (int i = w; i < n; i += 16) {
            // the row's loads first, with the column clamped into [i, n)
            // (lanes outside the triangle read S_ii or S_i,n-1, one cache
            // line, and discard it): no branches, so no load waits on the
            // one before it
            // (in batches of up to 8 blocks, for the registers)
            constexpr int NB = NM < 8 ? NM : 8;
            const TM* row = S + (int64_t)i * ld;
            const double vi = L.v1[i];
            double acc = 0.0;
#pragma unroll
            for (int m0 = 0; m0 < NM; m0 += NB) {
                TM sv[NB];
#pragma unroll
                for (int q = 0; q < NB; ++q) sv[q] = row[min(max(l + 64 * (m0 + q), i), n - 1)];
#pragma unroll
                for (int q = 0; q < NB; ++q) {
                    const int m = m0 + q, j = l + 64 * m;
                    const double sij = (j >= i && j < n) ? (double)sv[q] : 0.0;
                    acc += sij * vr[m];
                    wc[m] += (j > i) ? sij * vi : 0.0;
                }
            }
            const double x = wave_sum(acc);
            if (l == 0) L.wv[i] = x;
        }
#pragma unroll
        for (int m = 0; m < NM; ++m)
            if (l + 64 * m < n) L.part[w * kLanczosMaxN + l + 64 * m] = wc[m];
        __syncthreads();
        // w_j = (row part) + the sixteen waves' column parts, in wave order
        double d = 0.0;
        for (int j = t; j < n; j += 1024) {
            double cs = 0.0;
#pragma unroll
            for (int q = 0; q < 16; ++q) cs += L.part[q * kLanczosMaxN + j];
            const double wj = L.wv[j] + cs;
            L.wv[j] = wj;
            d += wj * L.v1[j];
        }
        const double alpha = block_sum_1024(d, L.red);
        double q = 0.0;
        for (int j = t; j < n; j += 1024) {
            const double x = L.wv[j] - alpha * L.v1[j] - beta_prev * L.v0[j];
            L.wv[j] = x;
            q += x * x;
        }
        const double beta = sqrt(block_sum_1024(q, L.red));
        if (t == 0) { L.al[k] = alpha; L.be[k] = beta; }
        const bool stop = !(beta > 1e-13 * fabs(alpha)) || !isfinite(alpha) || !isfinite(beta);
        if (stop) {
            if (t == 0) L.m_used = k + 1;
            __syncthreads();
            break;
        }
        if (args.tol > 0.0 && k + 1 < steps && lanczos_check_step(k + 1)) {
            __syncthreads();   // al, be of this step written
            if (w == 0) {
                const double th = tridiag_max_wave(L.al, L.be, k + 1);
                const double rs = ritz_residual(L.al, L.be, k + 1, th);
                if (l == 0) {
                    L.rstop = !(rs > args.tol * th);
                    if (L.rstop) L.m_used = k + 1;
                }
            }
            __syncthreads();
            if (L.rstop) break;   // uniform
        }
        for (int j = t; j < n; j += 1024) {
            L.v0[j] = L.v1[j];
            L.v1[j] = L.wv[j] / beta;
        }
        beta_prev = beta;
        __syncthreads();
    }
    __syncthreads();
    if (w == 0) {
        const double lm = tridiag_max_wave(L.al, L.be, L.m_used);
        if (l == 0) lanczos_finish(args, jb, isfinite(lm), lm);
    }
}

// The same Lanczos iteration for a few factors of 129..1024, split over
// launches so that one factor's product S v runs on many workgroups: per
// step, k_lz_matvec (one workgroup per 64 rows of a factor, each row summed
// exactly as in k_lanczos_big) and k_lz_update (one workgroup per factor:
// alpha, beta, the next vector); the vectors and the tridiagonal live in a
// per-factor work record.  The arithmetic, and so the result, is that of
// k_lanczos_big.
constexpr int kLzV0 = 0, kLzV1 = kLanczosMaxN, kLzW = 2 * kLanczosMaxN, kLzAl = 3 * kLanczosMaxN,
              kLzBe = kLzAl + kLanczosMaxSteps, kLzMisc = kLzBe + kLanczosMaxSteps;
// misc: [0] beta of the previous step, [1] steps used, [2] stopped flag
static_assert(kLzMisc + 3 <= kLzWork, "Lanczos work record");

__global__ __launch_bounds__(1024) void k_lz_start(const LanczosJob* __restrict__ jobs,
                                                  double* __restrict__ work, int steps_max) {
    __shared__ double red[16];
    const LanczosJob jb = jobs[blockIdx.x];
    double* wk = work + (int64_t)blockIdx.x * kLzWork;
    const int n = jb.n, t = threadIdx.x;
    double s2 = 0.0;
    for (int i = t; i < n; i += 1024) {
        uint32_t hsh = (uint32_t)i * 2654435761u + 0x9E3779B9u;
        hsh ^= hsh >> 15; hsh *= 2246822519u; hsh ^= hsh >> 13;
        const double x = 0.5 + (double)(hsh & 0xFFFFFF) / 16777216.0;
        wk[kLzV1 + i] = x;
        wk[kLzV0 + i] = 0.0;
        s2 += x * x;
    }
    const double inv = 1.0 / sqrt(block_sum_1024(s2, red));
    for (int i = t; i < n; i += 1024) wk[kLzV1 + i] *= inv;
    if (t == 0) {
        wk[kLzMisc] = 0.0;
        wk[kLzMisc + 1] = (double)min(steps_max, min(n, kLanczosMaxSteps));
        wk[kLzMisc + 2] = 0.0;
    }
}

template <typename TM>
__global__ __launch_bounds__(256) void k_lz_matvec(const LanczosJob* __restrict__ jobs,
                                                  const TM* __restrict__ arena,
                                                  double* __restrict__ work, int k) {
    const LanczosJob jb = jobs[blockIdx.y];
    double* wk = work + (int64_t)blockIdx.y * kLzWork;
    const int n = jb.n, ld = jb.ld;
    if (wk[kLzMisc + 2] != 0.0 || k >= (int)wk[kLzMisc + 1]) return;   // uniform
    const int r0 = 64 * blockIdx.x;
    if (r0 >= n) return;
    const TM* S = arena + jb.off;
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    double vr[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) vr[m] = (l + 64 * m < n) ? wk[kLzV1 + l + 64 * m] : 0.0;
    for (int i0 = r0 + w; i0 < r0 + 64 && i0 < n; i0 += 16) {
        double acc[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            acc[r] = 0.0;
            const int i = i0 + 4 * r;
            if (i < n && i < r0 + 64) {   // uniform
                // columns past n clamped to n - 1 (their v entry is 0): no
                // branches around the loads, so they are all in flight at once
                const TM* row = S + (int64_t)i * ld;
#pragma unroll
                for (int m = 0; m < 16; ++m) acc[r] += (double)row[min(l + 64 * m, n - 1)] * vr[m];
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const double x = wave_sum(acc[r]);
            const int i = i0 + 4 * r;
            if (l == 0 && i < n && i < r0 + 64) wk[kLzW + i] = x;
        }
    }
}

__global__ __launch_bounds__(1024) void k_lz_update(const LanczosJob* __restrict__ jobs,
                                                   double* __restrict__ work, int k, double tol) {
    __shared__ double red[16];
    __shared__ int rstop;
    const LanczosJob jb = jobs[blockIdx.x];
    double* wk = work + (int64_t)blockIdx.x * kLzWork;
    const int n = jb.n, t = threadIdx.x;
    if (wk[kLzMisc + 2] != 0.0 || k >= (int)wk[kLzMisc + 1]) return;   // uniform
    const double beta_prev = wk[kLzMisc];
    double d = 0.0;
    for (int j = t; j < n; j += 1024) d += wk[kLzW + j] * wk[kLzV1 + j];
    const double alpha = block_sum_1024(d, red);
    double q = 0.0;
    for (int j = t; j < n; j += 1024) {
        const double x = wk[kLzW + j] - alpha * wk[kLzV1 + j] - beta_prev * wk[kLzV0 + j];
        wk[kLzW + j] = x;
        q += x * x;
    }
    const double beta = sqrt(block_sum_1024(q, red));
    const bool stop = !(beta > 1e-13 * fabs(alpha)) || !isfinite(alpha) || !isfinite(beta);
    if (t == 0) {
        wk[kLzAl + k] = alpha;
        wk[kLzBe + k] = beta;
        if (stop) {
            wk[kLzMisc + 1] = (double)(k + 1);
            wk[kLzMisc + 2] = 1.0;
        }
        wk[kLzMisc] = beta;
    }
    if (stop) return;
    if (tol > 0.0 && k + 1 < (int)wk[kLzMisc + 1] && lanczos_check_step(k + 1)) {
        __syncthreads();   // this step's al, be written (same workgroup)
        if (t < 64) {
            const double th = tridiag_max_wave(wk + kLzAl, wk + kLzBe, k + 1);
            const double rs = ritz_residual(wk + kLzAl, wk + kLzBe, k + 1, th);
            if (t == 0) {
                rstop = !(rs > tol * th);
                if (rstop) {
                    wk[kLzMisc + 1] = (double)(k + 1);
                    wk[kLzMisc + 2] = 1.0;
                }
            }
        }
        __syncthreads();
        if (rstop) return;   // uniform
    }
    for (int j = t; j < n; j += 1024) {
        wk[kLzV0 + j] = wk[kLzV1 + j];
        wk[kLzV1 + j] = wk[kLzW + j] / beta;
    }
}

__global__ __launch_bounds__(64) void k_lz_finish(const LanczosJob* __restrict__ jobs,
                                                 const double* __restrict__ work, LanczosArgs args) {
    const LanczosJob jb = jobs[blockIdx.x];
    const double* wk = work + (int64_t)blockIdx.x * kLzWork;
    const double lm = tridiag_max_wave(wk + kLzAl, wk + kLzBe, (int)wk[kLzMisc + 1]);
    if (threadIdx.x == 0) lanczos_finish(args, jb, isfinite(lm), lm);
}

// ======================================================= coupled Newton
// Packs, per class of the gated fp64 chain (one workgroup each), the factors
// whose precision flag equals gate_val into the leading slots of the class in
// class order (a ballot prefix sum per pass of 1024 factors).  Slot k gets
// the factor's job with the scratch place k mod cap of its chunk and flag 1;
// the slots past the count get factor -1 (the chain's start and finish skip
// them) and flag 0 (its products skip them).
__global__ __launch_bounds__(1024) void k_route_compact(const CompactClass* __restrict__ cls,
                                                       const FactorJob* __restrict__ tmpl,
                                                       const int32_t* __restrict__ prec, int gate_val,
                                                       FactorJob* __restrict__ slots,
                                                       int32_t* __restrict__ live) {
    __shared__ int wtot[16];
    const CompactClass c = cls[blockIdx.x];
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    int carry = 0;
    for (int base = 0; base < c.n; base += 1024) {
        const int i = base + t;
        FactorJob j{};
        bool f = false;
        if (i < c.n) {
            j = tmpl[c.first + i];
            f = prec[j.factor] == gate_val;
        }
        const unsigned long long m = __ballot(f);
        if (lane == 0) wtot[w] = __popcll(m);
        __syncthreads();
        int before = carry, tot = 0;
        for (int q = 0; q < 16; ++q) {
            before += q < w ? wtot[q] : 0;
            tot += wtot[q];
        }
        if (f) {
            const int k = before + __popcll(m & ((1ull << lane) - 1ull));
            j.x_off = (int64_t)(k % c.cap) * 6 * c.mat;
            j.m_off = j.x_off + 2 * c.mat;
            slots[c.first + k] = j;
            live[c.first + k] = 1;
        }
        carry += tot;
        __syncthreads();   // wtot is rewritten by the next pass
    }
    for (int k = carry + t; k < c.n; k += 1024) {
        FactorJob j{};
        j.factor = -1;
        slots[c.first + k] = j;
        live[c.first + k] = 0;
    }
}

// Coupled Newton iteration for the inverse p-th root (Guo & Higham, SIAM J.
// Matrix Anal. Appl. 28(3), 2006).  With A = S + eps I (S read from its upper
// triangle) and z = (p+1) / (2 lambda_max(A)):  X_0 = z^(1/p) I, M_0 = z A; then
// T = ((p+1) I - M)/p, X <- X T, M <- T^p M.  M_k = X_k^p A throughout, so
// M -> I and X -> A^(-1/p).  Padded rows/columns carry M = I, X = I and stay
// decoupled (block diagonal).
// The 32 x 32 tiles (ti, tj) of a factor (blockIdx.y) are shared out over
// gridDim.x workgroups (tile = blockIdx.x + k gridDim.x); each thread takes 4
// consecutive columns of one row of a tile.  The statistic is read from its
// upper triangle: a tile below the diagonal reads its mirror tile
// (coalesced) and transposes it in LDS.  X_0 is diagonal, so the first
// product X_1 = X_0 T(M_0) is a row scaling: the start writes X_1 (into the
// second X buffer) and the chain's first iteration skips that product.
template <typename T>
__global__ __launch_bounds__(256) void k_newton_init(const FactorJob* __restrict__ jobs,
                                                    const double* __restrict__ stats,
                                                    T* __restrict__ scratch,
                                                    const FactorDiag* __restrict__ diag,
                                                    NewtonArgs args) {
    __shared__ double ts[32][33];
    const FactorJob jb = jobs[blockIdx.y];
    if (jb.factor < 0 || (args.gate && args.gate[jb.factor] != args.gate_val)) return;
    const int n = jb.n, ld = jb.ld, nt = ld >> 5;
    if (blockIdx.x == 0 && threadIdx.x == 0) {   // the finish's check slots of this pass
        args.chk[2 * jb.factor] = 0ull;
        args.chk[2 * jb.factor + 1] = 0ull;
    }
    const FactorDiag dg = diag[jb.factor];
    const bool ok = dg.status == 0;
    const double lam = dg.lambda_max + dg.eps;
    const T z = ok ? T((args.p + 1) / (2.0 * lam)) : T(1);
    const T zr = ok ? T(pow((args.p + 1) / (2.0 * lam), 1.0 / args.p)) : T(1);
    const T e = T(dg.eps);
    const double* S = stats + jb.s_off;
    T* X = scratch + jb.x_off + (int64_t)ld * ld;   // X_1, the buffer of iteration 1
    T* M = scratch + jb.m_off;
    const T c1 = T(args.xc1), c2 = T(args.xc2);   // the first step's T, as the product's loader
    const int r = threadIdx.x >> 3, c0 = (threadIdx.x & 7) * 4;
    for (int tile = blockIdx.x; tile < nt * nt; tile += gridDim.x) {
        const int ti = tile / nt, tj = tile % nt;
        const int br = ti <= tj ? ti : tj, bc = ti <= tj ? tj : ti;   // the upper tile
        __syncthreads();   // the previous tile's reads of ts are done
        if (ok) {
#pragma unroll
            for (int q = 0; q < 4; ++q) ts[r][c0 + q] = S[(int64_t)(32 * br + r) * ld + 32 * bc + c0 + q];
        }
        __syncthreads();
        const int i = 32 * ti + r;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int c = c0 + q, j = 32 * tj + c;
            T m, x;
            if (i < n && j < n && ok) {
                const int a = ti < tj ? r : (ti > tj ? c : min(r, c));
                const int b = ti < tj ? c : (ti > tj ? r : max(r, c));
                m = z * (T(ts[a][b]) + (i == j ? e : T(0)));
                // T(M_0) as the product's operand loader forms it, times z^(1/p)
                T tv = m * c2;
                if (i == j) tv += c1;
                x = zr * tv;
            } else {
                m = (i == j) ? T(1) : T(0);
                x = (i == j) ? T(1) : T(0);
            }
            M[(int64_t)i * ld + j] = m;
            X[(int64_t)i * ld + j] = x;
        }
    }
}

// Finish, part 1 (same sharing of tiles): max |M - I| of the last M formed
// (the one the last T came from) and whether X or M went
// non-finite, over the real n x n part, into the factor's check slots
// (atomic max of the bit patterns of non-negative doubles, which order like
// the values, so the result does not depend on the order).
template <typename T>
__global__ __launch_bounds__(256) void k_newton_check(const FactorJob* __restrict__ jobs,
                                                     const T* __restrict__ scratch,
                                                     const T* __restrict__ scratch_m,
                                                     const FactorDiag* __restrict__ diag,
                                                     NewtonArgs args) {
    __shared__ double red[4];
    const FactorJob jb = jobs[blockIdx.y];
    if (jb.factor < 0 || (args.gate && args.gate[jb.factor] != args.gate_val)) return;
    if (diag[jb.factor].status & (SHAMPOO_FACTOR_NONFINITE_INPUT_ | SHAMPOO_FACTOR_ZERO_)) return;
    const int n = jb.n, ld = jb.ld, nt = ld >> 5;
    const T* X = scratch + jb.x_off;
    const T* M = scratch_m + jb.m_off;
    const int r = threadIdx.x >> 3, c0 = (threadIdx.x & 7) * 4;
    double res = 0.0, bad = 0.0;
    for (int tile = blockIdx.x; tile < nt * nt; tile += gridDim.x) {
        const int ti = tile / nt, tj = tile % nt;
        const int i = 32 * ti + r;
        // every (i, j) < ld is inside the ld x ld buffers: the loads carry
        // no branches (all in flight at once) and the padding is masked after
        T xv[4], mv[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            xv[q] = X[(int64_t)i * ld + 32 * tj + c0 + q];
            mv[q] = M[(int64_t)i * ld + 32 * tj + c0 + q];
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int j = 32 * tj + c0 + q;
            if (i < n && j < n) {
                const double x = double(xv[q]);
                const double d = fabs(double(mv[q]) - (i == j ? 1.0 : 0.0));
                if (!isfinite(x) || !isfinite(d)) bad = 1.0;
                else res = fmax(res, d);
            }
        }
    }
    res = block_max_256(res, red);
    bad = block_max_256(bad, red);
    if (threadIdx.x == 0) {
        atomicMax(&args.chk[2 * jb.factor], (unsigned long long)__double_as_longlong(res));
        if (bad > 0.0) atomicMax(&args.chk[2 * jb.factor + 1], 1ull);
    }
}

// Finish, part 2 (same sharing of tiles): unless the factor's input or iterate went
// non-finite (then its previous root stays), the root is the symmetric part
// of X (the tile and its mirror, transposed in LDS), the identity for a
// factor with no statistics, identity on the padding; tile 0 records the
// status and the residual.
template <typename T>
__global__ __launch_bounds__(256) void k_newton_commit(const FactorJob* __restrict__ jobs,
                                                      float* __restrict__ arena,
                                                      const T* __restrict__ scratch,
                                                      FactorDiag* __restrict__ diag,
                                                      NewtonArgs args) {
    __shared__ double tm[32][33];
    const FactorJob jb = jobs[blockIdx.y];
    if (jb.factor < 0 || (args.gate && args.gate[jb.factor] != args.gate_val)) return;
    const int n = jb.n, ld = jb.ld, nt = ld >> 5;
    // status bits set before the iteration; this pass only adds others
    const int st0 = diag[jb.factor].status & (SHAMPOO_FACTOR_NONFINITE_INPUT_ | SHAMPOO_FACTOR_ZERO_);
    int st = st0;
    if (st0 == 0 && args.chk[2 * jb.factor + 1] != 0ull) st |= SHAMPOO_FACTOR_NONFINITE_ROOT_;
    const bool keep = (st & (SHAMPOO_FACTOR_NONFINITE_INPUT_ | SHAMPOO_FACTOR_NONFINITE_ROOT_)) != 0;
    const double res = st0 == 0 ? __longlong_as_double((long long)args.chk[2 * jb.factor]) : 0.0;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        FactorDiag& dg = diag[jb.factor];
        if (!keep && !(st & SHAMPOO_FACTOR_ZERO_) && res > 1e-2) st |= SHAMPOO_FACTOR_RESIDUAL_HIGH_;
        if (args.is_fp64) st |= SHAMPOO_FACTOR_FP64_;
        else st &= ~SHAMPOO_FACTOR_FP64_;
        dg.status = st;
        dg.residual = res;
        dg.iters = st0 == 0 ? args.iters : 0;
    }
    if (keep) return;
    const bool ident = (st & SHAMPOO_FACTOR_ZERO_) != 0;
    const T* X = scratch + jb.x_off;
    float* P = arena + jb.p_off;
    double* P64 = jb.p64_off >= 0 ? reinterpret_cast<double*>(arena) + jb.p64_off : nullptr;
    const int r = threadIdx.x >> 3, c0 = (threadIdx.x & 7) * 4;
    for (int tile = blockIdx.x; tile < nt * nt; tile += gridDim.x) {
        const int ti = tile / nt, tj = tile % nt;
        const int i = 32 * ti + r;
        // both tiles' values, inside the ld x ld buffer: loaded without
        // branches, all in flight at once (unused for an identity root)
        T xv[4], xt[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            xv[q] = X[(int64_t)i * ld + 32 * tj + c0 + q];
            xt[q] = X[(int64_t)(32 * tj + r) * ld + 32 * ti + c0 + q];
        }
        __syncthreads();   // the previous tile's reads of tm are done
#pragma unroll
        for (int q = 0; q < 4; ++q) tm[r][c0 + q] = double(xt[q]);
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int c = c0 + q, j = 32 * tj + c;
            double x;
            if (ident || i >= n || j >= n) x = (i == j) ? 1.0 : 0.0;
            else x = 0.5 * (double(xv[q]) + tm[c][r]);   // symmetric part
            P[(int64_t)i * ld + j] = float(x);
            if (P64) P64[(int64_t)i * ld + j] = x;
        }
    }
}

// ------------------------------------------- fused fp32 Newton, n <= 128
// The whole coupled iteration of one factor (padded to 128) in one workgroup
// of four waves, two workgroups per CU: the iterates live in registers as
// column strips (wave w owns columns [32w, 32w+32) of X, M and the powers of
// T, as four 32 x 32 MFMA accumulator tiles) and one LDS slot carries the
// left operand of each product.  The right operand is the wave's own strip,
// read straight from its registers: MFMA step (m', r) pairs the k-indices
// 32m' + 8(r/4) + r%4 and that + 4, exactly the two rows the accumulator
// layout keeps in register r of the two lane halves
// (v_mfma_f32_32x32x2f32: C lane l reg v = C[8(v/4) + 4(l/32) + v%4][l%32]).
// Per iteration (p = 4), with T = c1 I + c2 M: X' = c1 X + c2 X M (the same
// as X T), T2 = T T and T4 = T2 T2 (both operands from the slot), M' = T4 M.
// HBM is touched only to read S and to write P.
constexpr int kNP = 129;  // LDS pitch (floats) of the fused apply

struct CStrip {
    float v[4][16];   // v[m][r] = Y[32m + 8(r/4) + 4h + r%4][32w + c]
};

__device__ __forceinline__ int crow(int m, int h, int r) { return 32 * m + 8 * (r >> 2) + 4 * h + (r & 3); }

typedef float f16v __attribute__((ext_vector_type(16)));

// out = A B on the wave's column strip; A in the slot, bop(m', r) gives the
// right operand B[crow(m', h, r)][32w + c].  The 64 k-steps are fully
// unrolled (the right operand is indexed by register), with the four A
// values of step s+1 loaded before the MFMAs of step s and a scheduling
// barrier per step: the compiler may not hoist more loads, which keeps the
// three live strips (192 registers) within the 256 of two waves per SIMD.
// With B_FROM_SLOT the right operand is read from the slot as well.
template <bool B_FROM_SLOT, typename BF>
__device__ __forceinline__ void gemm_strip(const float* slot, BF&& bop, CStrip& out, int w, int h, int c) {
    f16v acc[4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[m][r] = 0.f;
    // lane (h, c) reads A[32m + c][k0 + 4h] at physical column pcol(k0) + 32h,
    // and B[k0 + 4h][32w + c]
    const float* Ar = slot + c * kSP + 32 * h;
    const float* Bc = slot + 4 * h * kSP + pcol(32 * w + c);
    auto kof = [](int s) { return 32 * (s >> 4) + 8 * ((s & 15) >> 2) + (s & 3); };
    float a[4], b;
#pragma unroll
    for (int m = 0; m < 4; ++m) a[m] = Ar[32 * m * kSP + pcol(kof(0))];
    if constexpr (B_FROM_SLOT) b = Bc[kof(0) * kSP];
#pragma unroll
    for (int s = 0; s < 64; ++s) {
        float an[4], bn = 0.f;
        if (s + 1 < 64) {
#pragma unroll
            for (int m = 0; m < 4; ++m) an[m] = Ar[32 * m * kSP + pcol(kof(s + 1))];
            if constexpr (B_FROM_SLOT) bn = Bc[kof(s + 1) * kSP];
        }
        const float bv = B_FROM_SLOT ? b : bop(s >> 4, s & 15);
#pragma unroll
        for (int m = 0; m < 4; ++m) acc[m] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[m], bv, acc[m], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (s + 1 < 64) {
#pragma unroll
            for (int m = 0; m < 4; ++m) a[m] = an[m];
            b = bn;
        }
    }
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int r = 0; r < 16; ++r) out.v[m][r] = acc[m][r];
}

template <typename BF>
__device__ __forceinline__ void gemm_slot_reg(const float* slot, BF&& bop, CStrip& out, int w, int h, int c) {
    gemm_strip<false>(slot, bop, out, w, h, c);
}

// out = A A with A in the slot (both operands read from LDS)
__device__ __forceinline__ void gemm_slot_slot(const float* slot, CStrip& out, int w, int h, int c) {
    gemm_strip<true>(slot, [](int, int) { return 0.f; }, out, w, h, c);
}

__device__ __forceinline__ void cstrip_store(float* slot, const CStrip& y, int w, int h, int c) {
    float* d = slot + 4 * h * kSP + pcol(32 * w + c);
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int r = 0; r < 16; ++r) d[(32 * m + 8 * (r >> 2) + (r & 3)) * kSP] = y.v[m][r];
}

// T = c1 I + c2 M into the slot from the wave's strip of M: c2 M everywhere,
// then the lane that owns the diagonal element of column col adds c1 (its own
// earlier write, so no barrier is needed in between).
__device__ __forceinline__ void store_newton_t(float* slot, const CStrip& M, float c1, float c2, int w,
                                               int h, int c) {
    float* d = slot + 4 * h * kSP + pcol(32 * w + c);
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int r = 0; r < 16; ++r) d[(32 * m + 8 * (r >> 2) + (r & 3)) * kSP] = c2 * M.v[m][r];
    if (((c >> 2) & 1) == h) {
        const int col = 32 * w + c;
        slot[sidx(col, col)] += c1;
    }
}

template <int PP>
__global__ __launch_bounds__(256, 2) void k_newton128(const FactorJob* __restrict__ jobs,
                                                     const double* __restrict__ stats,
                                                     float* __restrict__ arena,
                                                     FactorDiag* __restrict__ diag,
                                                     int32_t* __restrict__ prec, FusedArgs args) {
    __shared__ __align__(16) float slot[128 * kSP];
    __shared__ LanczosSlot lz;
    __shared__ double red[4];
    __shared__ double sh_lmax;   // re-read after the iteration: no set-up value lives across it
    __shared__ float sh_dev[4];  // per-wave sum of (M - I)^2 of the iterate just formed
    const FactorJob jb = jobs[blockIdx.x];
    const int n = jb.n, ld = jb.ld;
    constexpr int p = PP;
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int h = lane >> 5, c = lane & 31;
    const int col = 32 * w + c;

    // ---- S (fp64, upper triangle) -> slot, fp32, as the fp32 iteration sees it
    stage_sym(slot, stats + jb.s_off, n, ld);
    __syncthreads();

    // ---- lambda_max (Lanczos) -> eps, status
    auto setup = [&](double lm, int& st, bool& good, double& ep, double& la) {
        st = 0;
        if (!isfinite(lm)) st = SHAMPOO_FACTOR_NONFINITE_INPUT_;
        else if (!(lm > 0.0)) st = SHAMPOO_FACTOR_ZERO_;
        good = st == 0;
        ep = good ? args.eps_rel * lm : 0.0;
        la = lm + ep;
    };
    float z, zr, e;
    int iters;
    bool okp;
    {
        const double lm = lanczos_slot<true>(slot, n, args.steps_s, lz, args.lz_tol);
        if (t == 0) sh_lmax = lm;
        int st;
        double ep, la;
        setup(lm, st, okp, ep, la);
        z = okp ? float((p + 1) / (2.0 * la)) : 1.f;
        zr = okp ? float(pow((p + 1) / (2.0 * la), 1.0 / p)) : 1.f;
        e = float(ep);
        iters = okp ? args.iters : 0;
    }
    const float c1 = float((double)(p + 1) / p), c2 = float(-1.0 / p);

    // ---- M0 = z (S + eps I) in place in the slot (identity outside n x n),
    // read into the strips; then X0 = z^(1/p) I (identity outside n x n).
    // Element-wise passes run as rolled loops, so no per-element predicate
    // lives across the iteration.
    for (int e2 = t; e2 < 128 * 128; e2 += 256) {
        const int i = e2 >> 7, j = e2 & 127;
        float* q = slot + sidx(i, j);
        *q = (okp && i < n && j < n) ? z * (*q + (i == j ? e : 0.f)) : (i == j ? 1.f : 0.f);
    }
    __syncthreads();
    CStrip M;
    {
        const float* ms = slot + 4 * h * kSP + pcol(col);
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int r = 0; r < 16; ++r) M.v[m][r] = ms[(32 * m + 8 * (r >> 2) + (r & 3)) * kSP];
    }
    __syncthreads();
    for (int e2 = t; e2 < 128 * 128; e2 += 256) {
        const int i = e2 >> 7, j = e2 & 127;
        slot[sidx(i, j)] = (i == j) ? ((okp && i < n) ? zr : 1.f) : 0.f;
    }
    __syncthreads();

    // slot: X, registers: M.  X T = c1 X + c2 X M, so the first product takes
    // M itself as its right operand.
    // With a tolerance, the iteration ends one step after ||M - I||_F first
    // falls below it.  The Frobenius norm bounds the spectral one, and near I
    // the spectral error e maps to about (p+1)/(2p) e^2, so that step leaves
    // at most about tol^2: below fp32 resolution for tol <= 1e-3.
    const float tol = args.tol;
    int ran = iters;
    bool last = false;
    for (int it = 0; it < iters; ++it) {
        auto bM = [&](int mb, int r) { return M.v[mb][r]; };
        CStrip Xn;
        if (it == 0) {
            // X_0 is diagonal (z^(1/p) inside n x n, 1 outside), so X_0 M only
            // scales the rows of M (the product would add zeros to the same value)
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = 32 * m + 8 * (r >> 2) + 4 * h + (r & 3);
                    Xn.v[m][r] = slot[sidx(row, row)] * M.v[m][r];
                }
        } else {
            gemm_slot_reg(slot, bM, Xn, w, h, c);             // X M
        }
        {
            const float* xs = slot + 4 * h * kSP + pcol(col);
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    Xn.v[m][r] = fmaf(c2, Xn.v[m][r], c1 * xs[(32 * m + 8 * (r >> 2) + (r & 3)) * kSP]);
        }
        __syncthreads();
        store_newton_t(slot, M, c1, c2, w, h, c);
        __syncthreads();
        if constexpr (PP == 1) {
            gemm_slot_reg(slot, bM, M, w, h, c);              // M' = T M
        } else {
            // slot: Q = T^(p/2) by repeated squaring (p = 2: T itself), then
            // M' = Q (Q M): two products against register strips, so T^p
            // itself is never stored
#pragma unroll
            for (int e2 = 2; e2 < PP; e2 *= 2) {               // T^2, T^4
                CStrip Tp;
                gemm_slot_slot(slot, Tp, w, h, c);
                __syncthreads();
                cstrip_store(slot, Tp, w, h, c);
                __syncthreads();
            }
            CStrip Pm;
            gemm_slot_reg(slot, bM, Pm, w, h, c);             // Q M
            auto bP = [&](int mb, int r) { return Pm.v[mb][r]; };
            gemm_slot_reg(slot, bP, M, w, h, c);              // M' = Q (Q M)
        }
        __syncthreads();
        cstrip_store(slot, Xn, w, h, c);
        if (tol > 0.f) {
            // the diagonal tests are the same every step; an opaque column
            // keeps them from being hoisted out of the loop as 64 live masks
            int dcol = col;
            asm volatile("" : "+v"(dcol));
            float dv = 0.f;
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = 32 * m + 8 * (r >> 2) + 4 * h + (r & 3);
                    const float e = M.v[m][r] - (row == dcol ? 1.f : 0.f);
                    dv = fmaf(e, e, dv);
                }
            dv = wave_sum(dv);
            if (lane == 0) sh_dev[w] = dv;
        }
        __syncthreads();
        if (tol > 0.f) {
            // every thread reads the four values after the barrier above and
            // before the next step's first barrier, after which they are
            // written again: the exit is uniform over the workgroup
            if (last) {
                ran = it + 1;
                break;
            }
            last = (sh_dev[0] + sh_dev[1]) + (sh_dev[2] + sh_dev[3]) < tol * tol;
        }
    }

    // ---- commit.  Outside n x n both iterates hold the identity, so the
    // finiteness test and the residual run over the whole padded tile.
    const double lmax = sh_lmax;
    int st0;
    bool ok;
    double eps, lam;
    setup(lmax, st0, ok, eps, lam);
    double bad = 0.0;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            if (!isfinite(M.v[m][r])) bad = 1.0;
    for (int e2 = t; e2 < 128 * 128; e2 += 256)
        if (!isfinite(slot[e2 + (e2 >> 7)])) bad = 1.0;   // every stored element once
    bad = block_max_256(bad, red);
    int st = st0;
    if (ok && bad > 0.0) st |= SHAMPOO_FACTOR_NONFINITE_ROOT_;
    const bool keep = (st & (SHAMPOO_FACTOR_NONFINITE_INPUT_ | SHAMPOO_FACTOR_NONFINITE_ROOT_)) != 0;
    if (!keep) {
        // the committed root is the symmetric part (X + X^T)/2 (the exact root
        // is symmetric); identity outside n x n and for a zero factor
        const bool ident = (st & SHAMPOO_FACTOR_ZERO_) != 0;
        float* P = arena + jb.p_off;
        for (int e2 = t; e2 < ld * ld; e2 += 256) {
            const int i = e2 / ld, j = e2 - i * ld;
            const float xs = 0.5f * (slot[sidx(i, j)] + slot[sidx(j, i)]);
            P[e2] = (ident || i >= n || j >= n) ? ((i == j) ? 1.f : 0.f) : xs;
        }
    }

    // ---- kappa estimate from the root: lambda_max(X) = (lambda_min + eps)^(-1/p).
    // X is in the slot (identity block outside n x n, decoupled).
    double kap = 0.0;
    if (ok) {
        const double lx = lanczos_slot<true>(slot, n, args.steps_p, lz);
        if (isfinite(lx) && lx > 0.0) kap = lam * pow(lx, (double)p);
    }

    // ---- residual max |M - I|: M into the slot, the owner of each diagonal
    // element subtracts 1 from its own write
    double res = 0.0;
    if (ok) {
        __syncthreads();   // the slot (X) is no longer read
        cstrip_store(slot, M, w, h, c);
        if (((c >> 2) & 1) == h) slot[sidx(col, col)] -= 1.f;
        __syncthreads();
        for (int e2 = t; e2 < 128 * 128; e2 += 256) res = fmax(res, (double)fabsf(slot[e2 + (e2 >> 7)]));
        res = block_max_256(res, red);
    }
    if (!keep && !(st & SHAMPOO_FACTOR_ZERO_) && res > 1e-2) st |= SHAMPOO_FACTOR_RESIDUAL_HIGH_;
    if (t == 0) {
        FactorDiag& dg = diag[jb.factor];
        dg.lambda_max = lmax;
        dg.eps = eps;
        dg.kappa_est = kap;
        dg.status = st;
        dg.residual = ok ? res : 0.0;
        dg.iters = ok ? ran : 0;
        if (prec) {
            const bool weak = (st & (SHAMPOO_FACTOR_NONFINITE_ROOT_ | SHAMPOO_FACTOR_RESIDUAL_HIGH_)) != 0;
            prec[jb.factor] = (args.auto_route && ok && (kap > args.threshold || weak)) ? 1 : 0;
        }
    }
}

// --------------------------------------------------- fused apply, <= 128
// One block per workgroup of eight waves, one LDS tile (66 KB: two
// workgroups, sixteen waves per CU):
//  1. a <- a + G*G and ||A||^2 of A = G / (sqrt(a) + delta) while G is staged
//     into LDS (each thread: four rows of 16-byte loads in flight);
//  2. T = G P_R: wave w takes column strip w%4 and row tiles 2(w/4), +1;
//     P_R streamed from L2 with an 8-step prefetch; T replaces G in LDS;
//  3. D = P_L T: wave w takes row strip w%4 and column tiles 2(w/4), +1; the
//     A operand is read down the columns of P_L -- the committed roots are
//     symmetric, so this is P_L itself -- again streamed with prefetch;
//  4. ||D||^2, then D written in the tensor's layout, or (fuse) the graft,
//     momentum and weight update applied in place from D staged in LDS.
// Apply, graft and update of one block of at most 128 x 128 on a 512-thread
// workgroup; Sl: 128 x kNP floats of LDS, red: 8 doubles.
__device__ __forceinline__ void apply128_block(const ApplyJob& job, const uint64_t* __restrict__ bases,
                                               float* __restrict__ arena, float delta,
                                               double* __restrict__ partA, double* __restrict__ partD,
                                               const UpdateArgs& ua, float* Sl, double* red) {
    const ApplyJob jb = job;
    const float* G = base_ptr<const float>(bases, jb.g_base, jb.g_off);
    float* a = arena + jb.a_off;
    const int mb = jb.mb, nb = jb.nb, ld = jb.ldg;
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int h = lane >> 5, c = lane & 31;
    const int c4 = t & 31, r0 = t >> 5, cc = 4 * c4;   // elementwise: 16 rows per pass

    // ---- 1. G -> LDS with the Adagrad accumulate on the way
    double asum = 0.0;
    {
        const bool vec = (nb % 4 == 0) && (ld % 4 == 0) && ((reinterpret_cast<uintptr_t>(G) & 15) == 0) &&
                         ((reinterpret_cast<uintptr_t>(a) & 15) == 0);
        if (vec) {
#pragma unroll
          for (int u0 = 0; u0 < 8; u0 += 4) {
            float4 g4[4], a4[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int r = r0 + 16 * (u0 + u);
                g4[u] = make_float4(0.f, 0.f, 0.f, 0.f);
                a4[u] = g4[u];
                if (r < mb && cc < nb) {
                    g4[u] = *reinterpret_cast<const float4*>(G + (int64_t)r * ld + cc);
                    a4[u] = *reinterpret_cast<const float4*>(a + (int64_t)r * ld + cc);
                }
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int r = r0 + 16 * (u0 + u);
                const float4 gv = g4[u];
                if (r < mb && cc < nb) {
                    float4 av = a4[u];
                    av.x += gv.x * gv.x; av.y += gv.y * gv.y; av.z += gv.z * gv.z; av.w += gv.w * gv.w;
                    *reinterpret_cast<float4*>(a + (int64_t)r * ld + cc) = av;
                    const float A0 = gv.x / (sqrtf(av.x) + delta), A1 = gv.y / (sqrtf(av.y) + delta);
                    const float A2 = gv.z / (sqrtf(av.z) + delta), A3 = gv.w / (sqrtf(av.w) + delta);
                    asum += (double)(A0 * A0 + A1 * A1) + (double)(A2 * A2 + A3 * A3);
                }
                float* d = &Sl[r * kNP + cc];
                d[0] = gv.x; d[1] = gv.y; d[2] = gv.z; d[3] = gv.w;
            }
          }
        } else {
            for (int u = 0; u < 8; ++u) {
                const int r = r0 + 16 * u;
                float gv[4] = {0.f, 0.f, 0.f, 0.f};
                if (r < mb) {
                    for (int e = 0; e < 4 && cc + e < nb; ++e) {
                        const int64_t o = (int64_t)r * ld + cc + e;
                        const float g1 = G[o];
                        const float av = a[o] + g1 * g1;
                        a[o] = av;
                        const float A = g1 / (sqrtf(av) + delta);
                        asum += (double)(A * A);
                        gv[e] = g1;
                    }
                }
                float* d = &Sl[r * kNP + cc];
                d[0] = gv[0]; d[1] = gv[1]; d[2] = gv[2]; d[3] = gv[3];
            }
        }
    }
    __syncthreads();

    const int st = w & 3, hv = w >> 2;     // strip and half of this wave
    // ---- 2. T[32(2hv+r').., 32st..] = G[rows, :] P_R[:, 32st..]; k runs over
    // the first nb (rounded up to 16; beyond nb, P_R reads as zero)
    const int KT = (nb + 15) & ~15;
    const float* PR = arena + jb.pr_off;
    const int colT = 32 * st + c;          // this lane's column of P_R / T
    f16v tacc[2];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int v = 0; v < 16; ++v) tacc[r][v] = 0.f;
    {
        auto ld_pr = [&](int k) -> float {
            return (k < nb && colT < nb) ? PR[(int64_t)k * jb.ld_r + colT] : 0.f;
        };
        float nxt[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) nxt[u] = ld_pr(2 * u + h);
        for (int k0 = 0; k0 < KT; k0 += 16) {
            float cur[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) cur[u] = nxt[u];
            if (k0 + 16 < KT) {
#pragma unroll
                for (int u = 0; u < 8; ++u) nxt[u] = ld_pr(k0 + 16 + 2 * u + h);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int k = k0 + 2 * u + h;
#pragma unroll
                for (int r = 0; r < 2; ++r)
                    tacc[r] = __builtin_amdgcn_mfma_f32_32x32x2f32(Sl[(32 * (2 * hv + r) + c) * kNP + k],
                                                                   cur[u], tacc[r], 0, 0, 0);
            }
        }
    }
    __syncthreads();                       // every wave is done reading G
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int v = 0; v < 16; ++v)
            Sl[(32 * (2 * hv + r) + 8 * (v >> 2) + 4 * h + (v & 3)) * kNP + 32 * st + c] = tacc[r][v];
    __syncthreads();

    // ---- 3. D[32st.., 32(2hv+q')..] = P_L[32st.., :] T; A operand
    // P_L[32st + c][k] = P_L[k][32st + c] (symmetric), k over the first mb
    const int KD = (mb + 15) & ~15;
    const float* PL = arena + jb.pl_off;
    const int rowD = 32 * st + c;
    f16v dacc[2];
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int v = 0; v < 16; ++v) dacc[q][v] = 0.f;
    {
        auto ld_pl = [&](int k) -> float {
            return (k < mb && rowD < mb) ? PL[(int64_t)k * jb.ld_l + rowD] : 0.f;
        };
        float nxt[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) nxt[u] = ld_pl(2 * u + h);
        for (int k0 = 0; k0 < KD; k0 += 16) {
            float cur[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) cur[u] = nxt[u];
            if (k0 + 16 < KD) {
#pragma unroll
                for (int u = 0; u < 8; ++u) nxt[u] = ld_pl(k0 + 16 + 2 * u + h);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int k = k0 + 2 * u + h;
#pragma unroll
                for (int q = 0; q < 2; ++q)
                    dacc[q] = __builtin_amdgcn_mfma_f32_32x32x2f32(cur[u], Sl[k * kNP + 32 * (2 * hv + q) + c],
                                                                   dacc[q], 0, 0, 0);
            }
        }
    }

    // ---- 4. ||D||^2; then either D to memory (the graft scale needs every
    // block's norms first) or, for a block whose tensor is covered by such
    // blocks only, the graft, momentum and weight update right here: the
    // block's ||A||^2 and ||D||^2 are complete in this workgroup.
    double dsum = 0.0;
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int i = 32 * st + 8 * (v >> 2) + 4 * h + (v & 3), j = 32 * (2 * hv + q) + c;
            if (i < mb && j < nb) dsum += (double)dacc[q][v] * (double)dacc[q][v];
        }
    asum = block_sum_512(asum, red);
    dsum = block_sum_512(dsum, red);
    if (t == 0) {
        partA[jb.slot_a] = asum;
        partD[jb.slot_d] = dsum;
    }
    if (jb.fuse) {
        const float sc = dsum > 0.0 ? (float)sqrt(asum / dsum) : 0.f;   // as in k_block_scale
        float* W = base_ptr<float>(bases, jb.w_base, jb.g_off);
        float* mo = arena + jb.m_off;
        const float b1 = ua.beta1, lr = ua.lr;
        // D through LDS (T is no longer read after the barrier), then the
        // update in row-major order with 16-byte accesses, four rows of loads
        // in flight before their stores
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                Sl[(32 * st + 8 * (v >> 2) + 4 * h + (v & 3)) * kNP + 32 * (2 * hv + q) + c] = dacc[q][v];
        __syncthreads();
        const bool vec = (nb % 4 == 0) && (ld % 4 == 0) && ((reinterpret_cast<uintptr_t>(W) & 15) == 0) &&
                         ((reinterpret_cast<uintptr_t>(mo) & 15) == 0);
        if (vec) {
#pragma unroll
          for (int u0 = 0; u0 < 8; u0 += 4) {
            float4 m4[4], w4[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int r = r0 + 16 * (u0 + u);
                if (r < mb && cc < nb) {
                    m4[u] = *reinterpret_cast<const float4*>(mo + (int64_t)r * ld + cc);
                    w4[u] = *reinterpret_cast<const float4*>(W + (int64_t)r * ld + cc);
                }
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int r = r0 + 16 * (u0 + u);
                if (r < mb && cc < nb) {
                    const float* d = &Sl[r * kNP + cc];
                    float4 m = m4[u], wv = w4[u];
                    m.x = b1 * m.x + sc * d[0]; m.y = b1 * m.y + sc * d[1];
                    m.z = b1 * m.z + sc * d[2]; m.w = b1 * m.w + sc * d[3];
                    wv.x -= lr * m.x; wv.y -= lr * m.y; wv.z -= lr * m.z; wv.w -= lr * m.w;
                    *reinterpret_cast<float4*>(mo + (int64_t)r * ld + cc) = m;
                    *reinterpret_cast<float4*>(W + (int64_t)r * ld + cc) = wv;
                }
            }
          }
        } else {
            for (int u = 0; u < 8; ++u) {
                const int r = r0 + 16 * u;
                if (r >= mb) continue;
                for (int e = 0; e < 4 && cc + e < nb; ++e) {
                    const int64_t o = (int64_t)r * ld + cc + e;
                    const float m = b1 * mo[o] + sc * Sl[r * kNP + cc + e];
                    mo[o] = m;
                    W[o] -= lr * m;
                }
            }
        }
    } else {
        float* Dg = arena + jb.d_off;
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int i = 32 * st + 8 * (v >> 2) + 4 * h + (v & 3), j = 32 * (2 * hv + q) + c;
                if (i < mb && j < nb) Dg[(int64_t)i * ld + j] = dacc[q][v];
            }
    }
}

__global__ __launch_bounds__(512, 4) void k_apply128(const ApplyJob* __restrict__ jobs,
                                                    const uint64_t* __restrict__ bases,
                                                    float* __restrict__ arena, float delta,
                                                    double* __restrict__ partA,
                                                    double* __restrict__ partD, UpdateArgs ua) {
    __shared__ __align__(16) float Sl[128 * kNP];
    __shared__ double red[8];
    apply128_block(jobs[blockIdx.x], bases, arena, delta, partA, partD, ua, Sl, red);
}

// ------------------------------------------------ fused step, blocks <= 128
// Statistics and apply of one block in one workgroup of sixteen waves, for a
// step without a root pass (the two then share only read-only inputs):
//  0. G and P_L staged into LDS by all waves (G zero outside mb x nb, P_L
//     zero outside mb x mb);
//  1. waves 0-7: a <- a + G*G and ||A||^2 (G from LDS, accumulator rows
//     loaded in phase 0), then L <- beta L + alpha G G^T and
//     R <- beta R + alpha G^T G on fp64 MFMA (the quadrant split of the
//     statistics kernel, one diagonal quadrant and one off-diagonal half per
//     SIMD) with the read-modify-write of the upper triangles; at the same
//     time waves 8-15: T = G P_R and D = P_L T on v_mfma_f32_16x16x4f32, wave
//     8+y owning columns [16y, 16y+16) of T and D.  T's strip is the right operand of the second product straight from
//     its accumulator registers: C lane l reg v = C[4(l/16) + v][l%16], so
//     register (m', v) holds rows 16m' + v + {0, 4, 8, 12} across the four
//     lane groups -- the four k-indices of one MFMA step;
//  2. momentum and weight loads issued, ||A||^2 and ||D||^2 (fixed order), D
//     into LDS;
//  3. graft, momentum and weight update (or D out for a tensor that also has
//     blocks > 128) by all waves, in row-major 16-byte accesses.
// Each SIMD holds two waves of each half, so the fp64 products of one half
// overlap the memory traffic of the other.
// Extra workgroups of the launch take row chunks of dense-Adagrad tensors
// (independent of the blocks: their G, a, mom and W are their own), spread
// through the grid: their streaming uses memory bandwidth the blocks leave
// idle, and the launch's last round of blocks is no longer half empty.
typedef float f4v __attribute__((ext_vector_type(4)));

template <int NT>
__device__ __forceinline__ void update_chunk(const RowChunk& ch, const uint64_t* __restrict__ bases,
                                             int n_tensors, float* __restrict__ arena,
                                             const float* __restrict__ scale, const UpdateArgs& args);

__global__ __launch_bounds__(1024) void k_step128(const StepJob* __restrict__ jobs, int njobs,
                                                 const RowChunk* __restrict__ fold, int n_tensors,
                                                 const uint64_t* __restrict__ bases,
                                                 float* __restrict__ arena, double alpha, double beta,
                                                 float delta, double* __restrict__ partA,
                                                 double* __restrict__ partD, UpdateArgs ua) {
    __shared__ __align__(16) float Gs[128 * kGP];
    __shared__ __align__(16) float Ps[128 * kGP];
    __shared__ double red[16];
    // the row chunks sit at every sp-th place of the grid (sp = grid / chunks,
    // so all fit), spreading their streaming over the launch; the other
    // places are the blocks in order
    int bid = blockIdx.x;
    {
        const int nfold = (int)gridDim.x - njobs;
        if (nfold > 0) {
            const int sp = (int)gridDim.x / nfold;
            const int q = bid / sp;
            if (bid % sp == sp - 1 && q < nfold) {
                update_chunk<1024>(fold[q], bases, n_tensors, arena, nullptr, ua);
                return;
            }
            bid -= min(nfold, (bid + 1) / sp);
        }
    }
    const StepJob sj = jobs[bid];
    const ApplyJob& jb = sj.ap;
    const float* G = base_ptr<const float>(bases, jb.g_base, jb.g_off);
    float* a = arena + jb.a_off;
    const int mb = jb.mb, nb = jb.nb, ld = jb.ldg;
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const bool vec = (nb % 4 == 0) && (ld % 4 == 0) && ((reinterpret_cast<uintptr_t>(G) & 15) == 0) &&
                     ((reinterpret_cast<uintptr_t>(a) & 15) == 0);

    // ---- 0. G and P_L into LDS (32 float4 per row, 32 rows per pass); the
    // statistics half (threads 0-511) also loads its eight rows of the Adagrad
    // accumulator (16 rows per pass) for the Adagrad pass that opens phase 1
    const int ac4 = t & 31, arr = (t >> 5) & 15, acc4 = 4 * ac4;
    float4 a4[8];
    if (w < 8 && vec) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int r = arr + 16 * u;
            if (r < mb && acc4 < nb) a4[u] = *reinterpret_cast<const float4*>(a + (int64_t)r * ld + acc4);
        }
    }
    {
        const int c4 = t & 31, r0 = t >> 5, cc = 4 * c4;
        const float* PL = arena + jb.pl_off;
        float4 gv[4], pv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int r = r0 + 32 * u;
            gv[u] = make_float4(0.f, 0.f, 0.f, 0.f);
            pv[u] = gv[u];
            if (r < mb && cc < nb) {
                if (vec) {
                    gv[u] = *reinterpret_cast<const float4*>(G + (int64_t)r * ld + cc);
                } else {
                    const float* gr = G + (int64_t)r * ld + cc;
                    gv[u].x = gr[0];
                    if (cc + 1 < nb) gv[u].y = gr[1];
                    if (cc + 2 < nb) gv[u].z = gr[2];
                    if (cc + 3 < nb) gv[u].w = gr[3];
                }
            }
            if (r < mb && cc < mb) {   // cc + 3 < ld_l: ld_l is a multiple of 32
                pv[u] = *reinterpret_cast<const float4*>(PL + (int64_t)r * jb.ld_l + cc);
                if (cc + 1 >= mb) pv[u].y = 0.f;
                if (cc + 2 >= mb) pv[u].z = 0.f;
                if (cc + 3 >= mb) pv[u].w = 0.f;
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int r = r0 + 32 * u;
            *reinterpret_cast<float4*>(&Gs[r * kGP + cc]) = gv[u];
            *reinterpret_cast<float4*>(&Ps[r * kGP + cc]) = pv[u];
        }
    }
    __syncthreads();

    // ---- 1.
    double asum = 0.0, dsum = 0.0;
    f4v dacc[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) dacc[m] = f4v{0.f, 0.f, 0.f, 0.f};
    const int i = lane & 15, g = lane >> 4;     // 16x16x4 lane coordinates
    const int y = w - 8, col = 16 * y + i;      // apply half: this lane's column of T and D
    if (w < 8) {
        // a <- a + G*G and ||A||^2 (G from LDS; the accumulator rows are in
        // flight since phase 0), while the apply half starts its products
        if (vec) {
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int r = arr + 16 * u;
                if (r < mb && acc4 < nb) {
                    const float4 gq = *reinterpret_cast<const float4*>(&Gs[r * kGP + acc4]);
                    float4 q = a4[u];
                    q.x += gq.x * gq.x; q.y += gq.y * gq.y; q.z += gq.z * gq.z; q.w += gq.w * gq.w;
                    *reinterpret_cast<float4*>(a + (int64_t)r * ld + acc4) = q;
                    const float A0 = gq.x / (sqrtf(q.x) + delta), A1 = gq.y / (sqrtf(q.y) + delta);
                    const float A2 = gq.z / (sqrtf(q.z) + delta), A3 = gq.w / (sqrtf(q.w) + delta);
                    asum += (double)(A0 * A0 + A1 * A1) + (double)(A2 * A2 + A3 * A3);
                }
            }
        } else {
            for (int u = 0; u < 8; ++u) {
                const int r = arr + 16 * u;
                if (r >= mb) continue;
                for (int e = 0; e < 4 && acc4 + e < nb; ++e) {
                    const int64_t o = (int64_t)r * ld + acc4 + e;
                    const float g1 = Gs[r * kGP + acc4 + e];
                    const float av = a[o] + g1 * g1;
                    a[o] = av;
                    const float A = g1 / (sqrtf(av) + delta);
                    asum += (double)(A * A);
                }
            }
        }
        // statistics: each diagonal quadrant of L and R on one wave (10 tiles),
        // each off-diagonal quadrant split over two (8 tiles each).  Waves w
        // and w + 4 share a SIMD, so each SIMD gets one diagonal quadrant and
        // one off-diagonal half: 18 tiles of fp64 MFMA work per SIMD.
        const int KL = (nb + 15) & ~15, KR = (mb + 15) & ~15;
        double* stats = reinterpret_cast<double*>(arena);
        double* L = stats + sj.l_off;
        double* R = stats + sj.r_off;
        switch (w) {
            case 0: gram_quadrant<true, false>(Gs, 0, 0, KL, L, jb.ld_l, mb, alpha, beta, i, g); break;
            case 1: gram_quadrant<true, false>(Gs, 1, 1, KL, L, jb.ld_l, mb, alpha, beta, i, g); break;
            case 2: gram_quadrant<true, true>(Gs, 0, 0, KR, R, jb.ld_r, nb, alpha, beta, i, g); break;
            case 3: gram_quadrant<true, true>(Gs, 1, 1, KR, R, jb.ld_r, nb, alpha, beta, i, g); break;
            case 4: gram_quadrant<false, false, 0, 2>(Gs, 0, 1, KL, L, jb.ld_l, mb, alpha, beta, i, g); break;
            case 5: gram_quadrant<false, false, 2, 4>(Gs, 0, 1, KL, L, jb.ld_l, mb, alpha, beta, i, g); break;
            case 6: gram_quadrant<false, true, 0, 2>(Gs, 0, 1, KR, R, jb.ld_r, nb, alpha, beta, i, g); break;
            default: gram_quadrant<false, true, 2, 4>(Gs, 0, 1, KR, R, jb.ld_r, nb, alpha, beta, i, g); break;
        }
    } else {
        // T[:, 16y..] = G P_R[:, 16y..]: A operand G[16m + i][k + g] from LDS,
        // B operand P_R[k + g][col] streamed with an 8-step prefetch
        f4v tacc[8];
#pragma unroll
        for (int m = 0; m < 8; ++m) tacc[m] = f4v{0.f, 0.f, 0.f, 0.f};
        {
            const float* PR = arena + jb.pr_off;
            const int KT = (nb + 3) & ~3;
            auto ld_pr = [&](int k) -> float {
                return (k < nb && col < nb) ? PR[(int64_t)k * jb.ld_r + col] : 0.f;
            };
            float nxt[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) nxt[u] = ld_pr(4 * u + g);
            for (int k0 = 0; k0 < KT; k0 += 32) {
                float cur[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) cur[u] = nxt[u];
                if (k0 + 32 < KT) {
#pragma unroll
                    for (int u = 0; u < 8; ++u) nxt[u] = ld_pr(k0 + 32 + 4 * u + g);
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int k = k0 + 4 * u;
                    if (k < KT) {
#pragma unroll
                        for (int m = 0; m < 8; ++m)
                            tacc[m] = __builtin_amdgcn_mfma_f32_16x16x4f32(Gs[(16 * m + i) * kGP + k + g], cur[u],
                                                                           tacc[m], 0, 0, 0);
                    }
                }
            }
        }
        // D[:, 16y..] = P_L T[:, 16y..]: step (m', v) takes k = 16m' + 4g + v in
        // lane group g; A operand P_L[16m + i][k] = P_L[k][16m + i] (symmetric)
#pragma unroll
        for (int mq = 0; mq < 8; ++mq) {
            if (16 * mq >= mb) break;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int k = 16 * mq + 4 * g + v;
                const float b = tacc[mq][v];
#pragma unroll
                for (int m = 0; m < 8; ++m)
                    dacc[m] = __builtin_amdgcn_mfma_f32_16x16x4f32(Ps[k * kGP + 16 * m + i], b, dacc[m], 0, 0, 0);
            }
        }
#pragma unroll
        for (int m = 0; m < 8; ++m)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int r = 16 * m + 4 * g + v;
                if (r < mb && col < nb) dsum += (double)dacc[m][v] * (double)dacc[m][v];
            }
    }

    // ---- 2. momentum and weight rows of phase 3 in flight (32 rows per pass,
    // four rows per thread), norms, D into LDS (G is no longer read past
    // these barriers)
    const int c4 = t & 31, r0 = t >> 5, cc = 4 * c4;
    float* W = base_ptr<float>(bases, jb.w_base, jb.g_off);
    float* mo = arena + jb.m_off;
    const bool vw = jb.fuse && vec && ((reinterpret_cast<uintptr_t>(W) & 15) == 0) &&
                    ((reinterpret_cast<uintptr_t>(mo) & 15) == 0);
    float4 m4[4], w4[4];
    if (vw) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int r = r0 + 32 * u;
            if (r < mb && cc < nb) {
                m4[u] = *reinterpret_cast<const float4*>(mo + (int64_t)r * ld + cc);
                w4[u] = *reinterpret_cast<const float4*>(W + (int64_t)r * ld + cc);
            }
        }
    }
    asum = block_sum_1024(asum, red);
    dsum = block_sum_1024(dsum, red);
    if (t == 0) {
        partA[jb.slot_a] = asum;
        partD[jb.slot_d] = dsum;
    }
    if (w >= 8) {
#pragma unroll
        for (int m = 0; m < 8; ++m)
#pragma unroll
            for (int v = 0; v < 4; ++v) Gs[(16 * m + 4 * g + v) * kGP + col] = dacc[m][v];
    }
    __syncthreads();

    // ---- 3. update (or D out)
    if (jb.fuse) {
        const float sc = dsum > 0.0 ? (float)sqrt(asum / dsum) : 0.f;   // as in k_block_scale
        const float b1 = ua.beta1, lr = ua.lr;
        if (vw) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int r = r0 + 32 * u;
                if (r < mb && cc < nb) {
                    const float4 d = *reinterpret_cast<const float4*>(&Gs[r * kGP + cc]);
                    float4 m = m4[u], wv = w4[u];
                    m.x = b1 * m.x + sc * d.x; m.y = b1 * m.y + sc * d.y;
                    m.z = b1 * m.z + sc * d.z; m.w = b1 * m.w + sc * d.w;
                    wv.x -= lr * m.x; wv.y -= lr * m.y; wv.z -= lr * m.z; wv.w -= lr * m.w;
                    *reinterpret_cast<float4*>(mo + (int64_t)r * ld + cc) = m;
                    *reinterpret_cast<float4*>(W + (int64_t)r * ld + cc) = wv;
                }
            }
        } else {
            for (int u = 0; u < 4; ++u) {
                const int r = r0 + 32 * u;
                if (r >= mb) continue;
                for (int e = 0; e < 4 && cc + e < nb; ++e) {
                    const int64_t o = (int64_t)r * ld + cc + e;
                    const float m = b1 * mo[o] + sc * Gs[r * kGP + cc + e];
                    mo[o] = m;
                    W[o] -= lr * m;
                }
            }
        }
    } else {
        float* Dg = arena + jb.d_off;
        for (int u = 0; u < 4; ++u) {
            const int r = r0 + 32 * u;
            if (r >= mb) continue;
            for (int e = 0; e < 4 && cc + e < nb; ++e) Dg[(int64_t)r * ld + cc + e] = Gs[r * kGP + cc + e];
        }
    }
}

// Copies inside the state buffer, one job per workgroup (snapshot of the
// statistics and roots of a root-pass part, and the swap of its new roots).
__global__ __launch_bounds__(256) void k_copy_jobs(const CopyJob* __restrict__ jobs,
                                                  unsigned char* __restrict__ arena) {
    const CopyJob jb = jobs[blockIdx.x];
    const float4* src = reinterpret_cast<const float4*>(arena + jb.src);
    float4* dst = reinterpret_cast<float4*>(arena + jb.dst);
    const int64_t n = jb.bytes / 16;
    for (int64_t e = threadIdx.x; e < n; e += 4 * 256) {
        float4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (e + 256 * u < n) v[u] = src[e + 256 * u];
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (e + 256 * u < n) dst[e + 256 * u] = v[u];
    }
}

// ====================================== one-sided statistics: split-K sum
// S <- beta S + alpha sum_c part_c on one 32 x 32 tile pair (bi <= bj) of a
// statistic whose product was split over the long dimension.  The partials
// are added in chunk order (fixed, so the result does not depend on the
// launch); the tile is written at (bi, bj) and its transpose at (bj, bi),
// and on a diagonal tile the lower half is the transpose of the upper half,
// so S stays exactly symmetric.  Partials and S beyond dim are not touched
// (the batched GEMM writes only i, j < dim of the upper 128 x 128 tiles,
// which contain every 32 x 32 pair bi <= bj).
__global__ __launch_bounds__(256) void k_sym_reduce(const SymReduceJob* __restrict__ jobs,
                                                   const TileRef* __restrict__ tiles,
                                                   double* __restrict__ arena, double alpha,
                                                   double beta) {
    __shared__ double T[32][33];
    const TileRef tr = tiles[blockIdx.x];
    const SymReduceJob jb = jobs[tr.task];
    const int bi = tr.tile / jb.tiles, bj = tr.tile % jb.tiles;
    const int r = threadIdx.x >> 3, c0 = (threadIdx.x & 7) * 4;
    const int i = bi * 32 + r, j0 = bj * 32 + c0;
    const int64_t mat = (int64_t)jb.ld * jb.ld;
    double* S = arena + jb.s_off;
    const double* P = arena + jb.part_off + (int64_t)i * jb.ld + j0;
    // ld is a multiple of 32, so the 4 columns are in the row (possibly padding)
    double2 v0 = make_double2(0.0, 0.0), v1 = make_double2(0.0, 0.0);
    if (i < jb.dim) {
        int c = 0;
        for (; c + 2 <= jb.nparts; c += 2) {
            const double2 a0 = *reinterpret_cast<const double2*>(P + c * mat);
            const double2 a1 = *reinterpret_cast<const double2*>(P + c * mat + 2);
            const double2 b0 = *reinterpret_cast<const double2*>(P + (c + 1) * mat);
            const double2 b1 = *reinterpret_cast<const double2*>(P + (c + 1) * mat + 2);
            v0.x += a0.x; v0.y += a0.y; v1.x += a1.x; v1.y += a1.y;
            v0.x += b0.x; v0.y += b0.y; v1.x += b1.x; v1.y += b1.y;
        }
        if (c < jb.nparts) {
            const double2 a0 = *reinterpret_cast<const double2*>(P + c * mat);
            const double2 a1 = *reinterpret_cast<const double2*>(P + c * mat + 2);
            v0.x += a0.x; v0.y += a0.y; v1.x += a1.x; v1.y += a1.y;
        }
        const double* So = S + (int64_t)i * jb.ld + j0;
        const double2 s0 = *reinterpret_cast<const double2*>(So);
        const double2 s1 = *reinterpret_cast<const double2*>(So + 2);
        v0.x = beta * s0.x + alpha * v0.x; v0.y = beta * s0.y + alpha * v0.y;
        v1.x = beta * s1.x + alpha * v1.x; v1.y = beta * s1.y + alpha * v1.y;
    }
    T[r][c0] = v0.x; T[r][c0 + 1] = v0.y; T[r][c0 + 2] = v1.x; T[r][c0 + 3] = v1.y;
    __syncthreads();
    // every read of S above (this tile and, for bi < bj, none of the mirror
    // tile) is done before the writes below
    if (bi == bj) {
        if (i < jb.dim)
            for (int e = 0; e < 4; ++e) {
                const int c = c0 + e;
                if (j0 + e < jb.dim) S[(int64_t)i * jb.ld + j0 + e] = r <= c ? T[r][c] : T[c][r];
            }
        return;
    }
    if (i < jb.dim)
        for (int e = 0; e < 4; ++e)
            if (j0 + e < jb.dim) S[(int64_t)i * jb.ld + j0 + e] = T[r][c0 + e];
    // transpose: row bj*32 + r, columns bi*32 + c0 .. + 3
    const int it = bj * 32 + r, jt = bi * 32 + c0;
    if (it < jb.dim)
        for (int e = 0; e < 4; ++e)
            if (jt + e < jb.dim) S[(int64_t)it * jb.ld + jt + e] = T[c0 + e][r];
}

// Split-K products of the batched Newton chain: C = sum of the parts, in part
// order, on one 32 x 32 tile pair (bi <= bj) of the symmetric product; the
// tile is written at (bi, bj) and its transpose at (bj, bi) (a diagonal tile's
// lower half from its upper half), over the whole padded ld x ld.
template <typename T>
__global__ __launch_bounds__(256) void k_split_sum(const SplitSumJob* __restrict__ jobs,
                                                  const TileRef* __restrict__ tiles,
                                                  T* __restrict__ base, const int32_t* __restrict__ gate,
                                                  int gate_val) {
    __shared__ T tt[32][33];
    const TileRef tr = tiles[blockIdx.x];
    const SplitSumJob jb = jobs[tr.task];
    if (gate && jb.gate >= 0 && gate[jb.gate] != gate_val) return;
    const int bi = tr.tile / jb.tiles, bj = tr.tile % jb.tiles;
    const int r = threadIdx.x >> 3, c0 = (threadIdx.x & 7) * 4;
    const int64_t mat = (int64_t)jb.ld * jb.ld;
    const T* P = base + jb.part_off + (int64_t)(bi * 32 + r) * jb.ld + bj * 32 + c0;
    T v[4] = {T(0), T(0), T(0), T(0)};
    for (int c = 0; c < jb.nparts; ++c) {   // 16-byte aligned: ld and c0 are multiples of 4
        const T* q = P + c * mat;
        if constexpr (sizeof(T) == 4) {
            const float4 a = *reinterpret_cast<const float4*>(q);
            v[0] += a.x; v[1] += a.y; v[2] += a.z; v[3] += a.w;
        } else {
            const double2 a = *reinterpret_cast<const double2*>(q);
            const double2 b = *reinterpret_cast<const double2*>(q + 2);
            v[0] += a.x; v[1] += a.y; v[2] += b.x; v[3] += b.y;
        }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) tt[r][c0 + e] = v[e];
    __syncthreads();
    T* C = base + jb.c_off;
    if (bi == bj) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int c = c0 + e;
            C[(int64_t)(bi * 32 + r) * jb.ld + bj * 32 + c] = r <= c ? tt[r][c] : tt[c][r];
        }
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            C[(int64_t)(bi * 32 + r) * jb.ld + bj * 32 + c0 + e] = tt[r][c0 + e];
            C[(int64_t)(bj * 32 + r) * jb.ld + bi * 32 + c0 + e] = tt[c0 + e][r];
        }
    }
}

// Identity roots for every factor (state initialisation).
__global__ __launch_bounds__(256) void k_set_identity(const FactorJob* __restrict__ jobs,
                                                     float* __restrict__ arena) {
    const FactorJob jb = jobs[blockIdx.x];
    const int ld = jb.ld;
    float* P = arena + jb.p_off;
    double* P64 = jb.p64_off >= 0 ? reinterpret_cast<double*>(arena) + jb.p64_off : nullptr;
    const int64_t nn = (int64_t)ld * ld;
    for (int64_t idx = threadIdx.x; idx < nn; idx += 256) {
        const bool d = (idx / ld) == (idx % ld);
        P[idx] = d ? 1.f : 0.f;
        if (P64) P64[idx] = d ? 1.0 : 0.0;
    }
}

// ================================================== elementwise: Adagrad
// a <- a + G*G over one run of rows of a Shampoo block and the partial
// ||A||^2 of A = G / (sqrt(a) + delta) for that run (fixed order).
__global__ __launch_bounds__(256) void k_adagrad_norm(const BlockChunk* __restrict__ chunks,
                                                     const uint64_t* __restrict__ bases,
                                                     float* __restrict__ arena, float delta,
                                                     double* __restrict__ partA) {
    __shared__ double red[4];
    const BlockChunk ch = chunks[blockIdx.x];
    const float* G = base_ptr<const float>(bases, 1 + ch.tensor, 0);
    float* a = arena + ch.a_off;
    const int64_t total = (int64_t)ch.nrows * ch.ncols;
    double acc = 0.0;
    const bool vec = (ch.ncols % 4 == 0) && (ch.cols % 4 == 0) && (ch.col0 % 4 == 0) &&
                     ((reinterpret_cast<uintptr_t>(G) & 15) == 0);
    if (vec) {
        const int c4 = ch.ncols / 4;
        const int64_t t4 = total / 4;
        for (int64_t e = threadIdx.x; e < t4; e += 256) {
            const int r = ch.row0 + (int)(e / c4);
            const int c = ch.col0 + 4 * (int)(e % c4);
            const int64_t idx = (int64_t)r * ch.cols + c;
            const float4 g = *reinterpret_cast<const float4*>(G + idx);
            float4 av = *reinterpret_cast<const float4*>(a + idx);
            av.x += g.x * g.x; av.y += g.y * g.y; av.z += g.z * g.z; av.w += g.w * g.w;
            *reinterpret_cast<float4*>(a + idx) = av;
            const float A0 = g.x / (sqrtf(av.x) + delta), A1 = g.y / (sqrtf(av.y) + delta);
            const float A2 = g.z / (sqrtf(av.z) + delta), A3 = g.w / (sqrtf(av.w) + delta);
            acc += (double)(A0 * A0 + A1 * A1) + (double)(A2 * A2 + A3 * A3);
        }
    } else {
        for (int64_t e = threadIdx.x; e < total; e += 256) {
            const int r = ch.row0 + (int)(e / ch.ncols);
            const int c = ch.col0 + (int)(e % ch.ncols);
            const int64_t idx = (int64_t)r * ch.cols + c;
            const float g = G[idx];
            const float av = a[idx] + g * g;
            a[idx] = av;
            const float A = g / (sqrtf(av) + delta);
            acc += (double)(A * A);
        }
    }
    const double s = block_sum_256(acc, red);
    if (threadIdx.x == 0) partA[ch.slot] = s;
}

// One wave per block: lane l sums partials l, l + 64, ... in order, then a
// fixed butterfly across the wave (a fixed order whatever the launch; one
// partial per side reduces to that partial exactly).
__global__ __launch_bounds__(256) void k_block_scale(const BlockNorms* __restrict__ bn, int nblocks,
                                                    const double* __restrict__ partA,
                                                    const double* __restrict__ partD,
                                                    float* __restrict__ scale) {
    const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int l = threadIdx.x & 63;
    if (b >= nblocks) return;   // uniform per wave
    const BlockNorms q = bn[b];
    double na = 0.0, nd = 0.0;
    for (int k = l; k < q.a_count; k += 64) na += partA[q.a_first + k];
    for (int k = l; k < q.d_count; k += 64) nd += partD[q.d_first + k];
    na = wave_sum(na);
    nd = wave_sum(nd);
    if (l == 0) scale[q.block] = nd > 0.0 ? (float)sqrt(na / nd) : 0.f;
}

// ================================================== elementwise: update
// Shampoo rows:  U = scale_b D;  dense-Adagrad rows: a += g^2, U = g/(sqrt(a)+delta).
// Then mom <- beta1 mom + U and W <- W - lr mom.
// One row chunk of the update on a workgroup of NT threads.
template <int NT>
__device__ __forceinline__ void update_chunk(const RowChunk& ch, const uint64_t* __restrict__ bases,
                                             int n_tensors, float* __restrict__ arena,
                                             const float* __restrict__ scale, const UpdateArgs& args) {
    const float* G = base_ptr<const float>(bases, 1 + ch.tensor, 0);
    float* W = base_ptr<float>(bases, 1 + n_tensors + ch.tensor, 0);
    float* a = arena + ch.a_off;
    float* mom = arena + ch.m_off;
    const float* D = arena + ch.d_off;
    const int64_t base = (int64_t)ch.row0 * ch.cols;
    const int64_t total = (int64_t)ch.nrows * ch.cols;
    const float b1 = args.beta1, lr = args.lr, dl = args.delta;
    const bool vec = (ch.cols % 4 == 0) && ((reinterpret_cast<uintptr_t>(W) & 15) == 0) &&
                     ((reinterpret_cast<uintptr_t>(G) & 15) == 0);
    if (vec && ch.mode == 0) {
        // Shampoo tensor: every load of kU 16-byte groups (D, momentum,
        // weight) issued before their stores, so each thread keeps 3 kU loads
        // in flight (the arrays do not alias, but the compiler cannot know)
        constexpr int kU = 4;
        const int64_t t4 = total / 4;
        const int c4 = ch.cols / 4;
        for (int64_t e0 = threadIdx.x; e0 < t4; e0 += NT * kU) {
            float4 d[kU], m[kU], w[kU];
            float sc[kU];
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                const int64_t e = e0 + NT * u;
                if (e < t4) {
                    const int64_t idx = base + 4 * e;
                    d[u] = *reinterpret_cast<const float4*>(D + idx);
                    m[u] = *reinterpret_cast<const float4*>(mom + idx);
                    w[u] = *reinterpret_cast<const float4*>(W + idx);
                    const int r = ch.row0 + (int)(e / c4);
                    const int c = 4 * (int)(e % c4);
                    sc[u] = scale[ch.first_block + (r / ch.block_size) * ch.nbc + c / ch.block_size];
                }
            }
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                const int64_t e = e0 + NT * u;
                if (e < t4) {
                    const int64_t idx = base + 4 * e;
                    const float s = sc[u];
                    const float4 uu = make_float4(s * d[u].x, s * d[u].y, s * d[u].z, s * d[u].w);
                    float4 mm = m[u], ww = w[u];
                    mm.x = b1 * mm.x + uu.x; mm.y = b1 * mm.y + uu.y;
                    mm.z = b1 * mm.z + uu.z; mm.w = b1 * mm.w + uu.w;
                    ww.x -= lr * mm.x; ww.y -= lr * mm.y; ww.z -= lr * mm.z; ww.w -= lr * mm.w;
                    *reinterpret_cast<float4*>(mom + idx) = mm;
                    *reinterpret_cast<float4*>(W + idx) = ww;
                }
            }
        }
    } else if (vec) {
        // dense Adagrad: the loads of kU groups (G, a, momentum, weight)
        // before their stores, as above
        constexpr int kU = 4;
        const int64_t t4 = total / 4;
        for (int64_t e0 = threadIdx.x; e0 < t4; e0 += NT * kU) {
            float4 g[kU], av[kU], m[kU], w[kU];
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                const int64_t e = e0 + NT * u;
                if (e < t4) {
                    const int64_t idx = base + 4 * e;
                    g[u] = *reinterpret_cast<const float4*>(G + idx);
                    av[u] = *reinterpret_cast<const float4*>(a + idx);
                    m[u] = *reinterpret_cast<const float4*>(mom + idx);
                    w[u] = *reinterpret_cast<const float4*>(W + idx);
                }
            }
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                const int64_t e = e0 + NT * u;
                if (e < t4) {
                    const int64_t idx = base + 4 * e;
                    float4 aa = av[u], mm = m[u], ww = w[u];
                    const float4 gg = g[u];
                    aa.x += gg.x * gg.x; aa.y += gg.y * gg.y; aa.z += gg.z * gg.z; aa.w += gg.w * gg.w;
                    const float4 uu = make_float4(gg.x / (sqrtf(aa.x) + dl), gg.y / (sqrtf(aa.y) + dl),
                                                  gg.z / (sqrtf(aa.z) + dl), gg.w / (sqrtf(aa.w) + dl));
                    mm.x = b1 * mm.x + uu.x; mm.y = b1 * mm.y + uu.y;
                    mm.z = b1 * mm.z + uu.z; mm.w = b1 * mm.w + uu.w;
                    ww.x -= lr * mm.x; ww.y -= lr * mm.y; ww.z -= lr * mm.z; ww.w -= lr * mm.w;
                    *reinterpret_cast<float4*>(a + idx) = aa;
                    *reinterpret_cast<float4*>(mom + idx) = mm;
                    *reinterpret_cast<float4*>(W + idx) = ww;
                }
            }
        }
    } else {
        for (int64_t e = threadIdx.x; e < total; e += NT) {
            const int64_t idx = base + e;
            float u;
            if (ch.mode == 0) {
                const int r = ch.row0 + (int)(e / ch.cols);
                const int c = (int)(e % ch.cols);
                const int blk = ch.first_block + (r / ch.block_size) * ch.nbc + c / ch.block_size;
                u = scale[blk] * D[idx];
            } else {
                const float g = G[idx];
                const float av = a[idx] + g * g;
                a[idx] = av;
                u = g / (sqrtf(av) + dl);
            }
            const float m = b1 * mom[idx] + u;
            mom[idx] = m;
            W[idx] -= lr * m;
        }
    }
}

__global__ __launch_bounds__(256) void k_update(const RowChunk* __restrict__ chunks,
                                               const uint64_t* __restrict__ bases, int n_tensors,
                                               float* __restrict__ arena,
                                               const float* __restrict__ scale, UpdateArgs args) {
    update_chunk<256>(chunks[blockIdx.x], bases, n_tensors, arena, scale, args);
}

// ============================= sparse-row tables, one-sided preconditioning
// The job of workgroup `chunk`: the last job whose first chunk is <= chunk
// (a handful of tables per call: a linear scan over the small table).
__device__ __forceinline__ int sos_job_of(const SosJob* __restrict__ jobs, int njobs, int chunk) {
    int j = 0;
    while (j + 1 < njobs && jobs[j + 1].first_chunk <= chunk) ++j;
    return j;
}

// On one chunk of a table's listed rows: a_r <- a_r + g*g and the partial
// ||A||^2 of A = g / (sqrt(a_r) + delta) (fixed order per chunk).
__global__ __launch_bounds__(256) void k_sos_norm(const SosJob* __restrict__ jobs, int njobs,
                                                 float* __restrict__ arena, float delta,
                                                 double* __restrict__ partA) {
    __shared__ double red[4];
    const SosJob jb = jobs[sos_job_of(jobs, njobs, blockIdx.x)];
    const int c = blockIdx.x - jb.first_chunk;
    const int64_t i0 = (int64_t)c * jb.chunk_rows;
    const int64_t i1 = i0 + jb.chunk_rows < jb.n_rows ? i0 + jb.chunk_rows : jb.n_rows;
    const int32_t* rows = global_ptr<const int32_t>(jb.rows_ptr);
    const float* G = global_ptr<const float>(jb.grads_ptr);
    float* a = arena + jb.a_off;
    const int cols = jb.cols;
    double acc = 0.0;
    if (jb.vec) {
        const int c4 = cols / 4;
        const int64_t total = (i1 - i0) * c4;
        for (int64_t e = threadIdx.x; e < total; e += 256) {
            const int64_t i = i0 + e / c4;
            const int q = (int)(e % c4);
            const int64_t r = rows[i];
            if (r < 0 || r >= jb.table_rows) continue;
            const float4 g = reinterpret_cast<const float4*>(G + i * cols)[q];
            float4* ap = reinterpret_cast<float4*>(a + r * cols) + q;
            float4 av = *ap;
            av.x += g.x * g.x; av.y += g.y * g.y; av.z += g.z * g.z; av.w += g.w * g.w;
            *ap = av;
            const float A0 = g.x / (sqrtf(av.x) + delta), A1 = g.y / (sqrtf(av.y) + delta);
            const float A2 = g.z / (sqrtf(av.z) + delta), A3 = g.w / (sqrtf(av.w) + delta);
            acc += (double)(A0 * A0 + A1 * A1) + (double)(A2 * A2 + A3 * A3);
        }
    } else {
        const int64_t total = (i1 - i0) * cols;
        for (int64_t e = threadIdx.x; e < total; e += 256) {
            const int64_t i = i0 + e / cols;
            const int q = (int)(e % cols);
            const int64_t r = rows[i];
            if (r < 0 || r >= jb.table_rows) continue;
            const float g = G[i * cols + q];
            const float av = a[r * cols + q] + g * g;
            a[r * cols + q] = av;
            const float A = g / (sqrtf(av) + delta);
            acc += (double)(A * A);
        }
    }
    const double s = block_sum_256(acc, red);
    if (threadIdx.x == 0) partA[jb.slot_a + c] = s;
}

// W_r <- W_r - lr s D_i for the listed rows (s the table's graft scale; no
// momentum, so rows that are not listed are not touched).
__global__ __launch_bounds__(256) void k_sos_update(const SosJob* __restrict__ jobs, int njobs,
                                                   const float* __restrict__ arena,
                                                   const float* __restrict__ scale, float lr) {
    const SosJob jb = jobs[sos_job_of(jobs, njobs, blockIdx.x)];
    const int c = blockIdx.x - jb.first_chunk;
    const int64_t i0 = (int64_t)c * jb.chunk_rows;
    const int64_t i1 = i0 + jb.chunk_rows < jb.n_rows ? i0 + jb.chunk_rows : jb.n_rows;
    const int32_t* rows = global_ptr<const int32_t>(jb.rows_ptr);
    const float* D = arena + jb.d_off;
    float* W = global_ptr<float>(jb.w_ptr);
    const float s = scale[jb.block];
    const int cols = jb.cols;
    if (jb.vec) {
        const int c4 = cols / 4;
        const int64_t total = (i1 - i0) * c4;
        for (int64_t e = threadIdx.x; e < total; e += 256) {
            const int64_t i = i0 + e / c4;
            const int q = (int)(e % c4);
            const int64_t r = rows[i];
            if (r < 0 || r >= jb.table_rows) continue;
            const float4 d = reinterpret_cast<const float4*>(D + i * cols)[q];
            float4* wp = reinterpret_cast<float4*>(W + r * cols) + q;
            float4 w = *wp;
            w.x -= lr * (s * d.x); w.y -= lr * (s * d.y); w.z -= lr * (s * d.z); w.w -= lr * (s * d.w);
            *wp = w;
        }
    } else {
        const int64_t total = (i1 - i0) * cols;
        for (int64_t e = threadIdx.x; e < total; e += 256) {
            const int64_t i = i0 + e / cols;
            const int q = (int)(e % cols);
            const int64_t r = rows[i];
            if (r < 0 || r >= jb.table_rows) continue;
            W[r * cols + q] -= lr * (s * D[i * cols + q]);
        }
    }
}

// ================================================ sparse-row Adagrad
__global__ __launch_bounds__(256) void k_sparse_rows(const SparseJob* __restrict__ jobs, int njobs,
                                                    int64_t total, float* __restrict__ arena,
                                                    float lr, float delta) {
    const int64_t item = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (item >= total) return;
    int j = 0;
    while (j + 1 < njobs && jobs[j + 1].first_item <= item) ++j;
    const SparseJob jb = jobs[j];
    const int64_t li = item - jb.first_item;
    const int32_t* rows = global_ptr<const int32_t>(jb.rows_ptr);
    const float* g = global_ptr<const float>(jb.grads_ptr);
    float* W = global_ptr<float>(jb.w_ptr);
    float* a = arena + jb.a_off;
    if (jb.vec) {
        const int c4 = jb.cols / 4;
        const int64_t k = li / c4;
        const int c = 4 * (int)(li % c4);
        const int64_t r = rows[k];
        if (r < 0 || r >= jb.table_rows) return;
        const float4 gv = *reinterpret_cast<const float4*>(g + k * jb.cols + c);
        float4 av = *reinterpret_cast<float4*>(a + r * jb.cols + c);
        float4 wv = *reinterpret_cast<float4*>(W + r * jb.cols + c);
        av.x += gv.x * gv.x; av.y += gv.y * gv.y; av.z += gv.z * gv.z; av.w += gv.w * gv.w;
        wv.x -= lr * gv.x / (sqrtf(av.x) + delta);
        wv.y -= lr * gv.y / (sqrtf(av.y) + delta);
        wv.z -= lr * gv.z / (sqrtf(av.z) + delta);
        wv.w -= lr * gv.w / (sqrtf(av.w) + delta);
        *reinterpret_cast<float4*>(a + r * jb.cols + c) = av;
        *reinterpret_cast<float4*>(W + r * jb.cols + c) = wv;
    } else {
        const int64_t k = li / jb.cols;
        const int c = (int)(li % jb.cols);
        const int64_t r = rows[k];
        if (r < 0 || r >= jb.table_rows) return;
        const float gv = g[k * jb.cols + c];
        const float av = a[r * jb.cols + c] + gv * gv;
        a[r * jb.cols + c] = av;
        W[r * jb.cols + c] -= lr * gv / (sqrtf(av) + delta);
    }
}

// ================================================================ launches
hipError_t launch_gemm_f32(const GemmTask* tasks, const TileRef* tiles, int ntiles,
                           const uint64_t* bases, const GemmArgs& a, hipStream_t s, int role) {
    if (ntiles <= 0) return hipSuccess;
    if (a.epi == EPI_AXPBY)
        hipLaunchKernelGGL((k_gemm<float, float, float, 1, true, false>), dim3(ntiles), dim3(256), 0, s,
                           tasks, tiles, bases, a);
    else if (role == 1)
        hipLaunchKernelGGL((k_gemm<float, float, float, 1, false, false, 1>), dim3(ntiles), dim3(256), 0,
                           s, tasks, tiles, bases, a);
    else if (role == 2)
        hipLaunchKernelGGL((k_gemm<float, float, float, 1, false, false, 2>), dim3(ntiles), dim3(256), 0,
                           s, tasks, tiles, bases, a);
    else
        hipLaunchKernelGGL((k_gemm<float, float, float, 3, false, false>), dim3(ntiles), dim3(256), 0, s,
                           tasks, tiles, bases, a);
    return hipGetLastError();
}
hipError_t launch_gemm_nt3(const NtTask* tasks, const TileRef* tiles, int ntiles,
                           const uint64_t* bases, const NtArgs& a, bool adagrad, hipStream_t s) {
    if (ntiles <= 0) return hipSuccess;
    if (adagrad)
        hipLaunchKernelGGL(k_gemm_nt3<true>, dim3(ntiles), dim3(256), 0, s, tasks, tiles, bases, a);
    else
        hipLaunchKernelGGL(k_gemm_nt3<false>, dim3(ntiles), dim3(256), 0, s, tasks, tiles, bases, a);
    return hipGetLastError();
}
hipError_t launch_gemm_f64(const GemmTask* tasks, const TileRef* tiles, int ntiles,
                           const uint64_t* bases, const GemmArgs& a, hipStream_t s) {
    if (ntiles <= 0) return hipSuccess;
    if (a.persist > 0 && a.epi != EPI_AXPBY) {
        GemmArgs b = a;
        b.ntiles = ntiles;
        const int groups = (ntiles + (a.chain > 1 ? a.chain : 1) - 1) / (a.chain > 1 ? a.chain : 1);
        hipLaunchKernelGGL((k_gemm<double, double, double, 2, false, true>),
                           dim3(groups < a.persist ? groups : a.persist), dim3(256), 0, s, tasks, tiles,
                           bases, b);
        return hipGetLastError();
    }
    if (a.epi == EPI_AXPBY)
        hipLaunchKernelGGL((k_gemm<double, double, double, 2, true, false>), dim3(ntiles), dim3(256), 0, s,
                           tasks, tiles, bases, a);
    else
        hipLaunchKernelGGL((k_gemm<double, double, double, 2, false, false>), dim3(ntiles), dim3(256), 0, s,
                           tasks, tiles, bases, a);
    return hipGetLastError();
}
hipError_t launch_gemm_f64_from_f32(const GemmTask* tasks, const TileRef* tiles, int ntiles,
                                    const uint64_t* bases, const GemmArgs& a, hipStream_t s) {
    if (ntiles <= 0) return hipSuccess;
    if (a.epi == EPI_AXPBY)
        hipLaunchKernelGGL((k_gemm<double, float, float, 2, true, false>), dim3(ntiles), dim3(256), 0, s,
                           tasks, tiles, bases, a);
    else
        hipLaunchKernelGGL((k_gemm<double, float, float, 2, false, false>), dim3(ntiles), dim3(256), 0, s,
                           tasks, tiles, bases, a);
    return hipGetLastError();
}
hipError_t launch_gram128(const GramJob* jobs, int njobs, const uint64_t* bases, double* stats,
                          double alpha, double beta, hipStream_t s) {
    if (njobs <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_gram128, dim3(njobs), dim3(512), 0, s, jobs, bases, stats, alpha, beta);
    return hipGetLastError();
}
hipError_t launch_lanczos(const LanczosJob* jobs, int njobs, const void* arena, bool fp64_matrix,
                          bool big, const LanczosArgs& a, hipStream_t s) {
    if (njobs <= 0) return hipSuccess;
    if (a.steps < 1) return hipErrorInvalidValue;
    if (big && njobs <= kLanczosSplitMax && a.work) {
        // few factors: the product of each step on many workgroups
        hipLaunchKernelGGL(k_lz_start, dim3(njobs), dim3(1024), 0, s, jobs, a.work, a.steps);
        const dim3 mv(kLanczosMaxN / 64, njobs);
        const int steps = std::min(a.steps, kLanczosMaxSteps);
        for (int k = 0; k < steps; ++k) {
            if (fp64_matrix)
                hipLaunchKernelGGL(k_lz_matvec<double>, mv, dim3(256), 0, s, jobs,
                                   static_cast<const double*>(arena), a.work, k);
            else
                hipLaunchKernelGGL(k_lz_matvec<float>, mv, dim3(256), 0, s, jobs,
                                   static_cast<const float*>(arena), a.work, k);
            hipLaunchKernelGGL(k_lz_update, dim3(njobs), dim3(1024), 0, s, jobs, a.work, k, a.tol);
        }
        hipLaunchKernelGGL(k_lz_finish, dim3(njobs), dim3(64), 0, s, jobs, a.work, a);
    } else if (big) {
        // 64-column blocks per row: the fewest that cover the largest factor
        const int nm = a.max_n > 0 && a.max_n <= 256 ? 4 : a.max_n > 0 && a.max_n <= 512 ? 8 : 16;
        auto go = [&](auto nmc) {
            constexpr int NM = decltype(nmc)::value;
            if (fp64_matrix)
                hipLaunchKernelGGL((k_lanczos_big<double, NM>), dim3(njobs), dim3(1024), 0, s, jobs,
                                   static_cast<const double*>(arena), a);
            else
                hipLaunchKernelGGL((k_lanczos_big<float, NM>), dim3(njobs), dim3(1024), 0, s, jobs,
                                   static_cast<const float*>(arena), a);
        };
        if (nm == 4) go(std::integral_constant<int, 4>{});
        else if (nm == 8) go(std::integral_constant<int, 8>{});
        else go(std::integral_constant<int, 16>{});
    } else {
        if (fp64_matrix)
            hipLaunchKernelGGL(k_lanczos<double>, dim3(njobs), dim3(256), 0, s, jobs,
                               static_cast<const double*>(arena), a);
        else
            hipLaunchKernelGGL(k_lanczos<float>, dim3(njobs), dim3(256), 0, s, jobs,
                               static_cast<const float*>(arena), a);
    }
    return hipGetLastError();
}
hipError_t launch_split_sum(bool fp64, const SplitSumJob* jobs, const TileRef* tiles, int ntiles,
                            void* arena, const int32_t* gate, int gate_val, hipStream_t s) {
    if (ntiles <= 0) return hipSuccess;
    if (fp64)
        hipLaunchKernelGGL(k_split_sum<double>, dim3(ntiles), dim3(256), 0, s, jobs, tiles,
                           static_cast<double*>(arena), gate, gate_val);
    else
        hipLaunchKernelGGL(k_split_sum<float>, dim3(ntiles), dim3(256), 0, s, jobs, tiles,
                           static_cast<float*>(arena), gate, gate_val);
    return hipGetLastError();
}
hipError_t launch_route_compact(const CompactClass* cls, int ncls, const FactorJob* tmpl,
                                const int32_t* prec, int gate_val, FactorJob* slots, int32_t* live,
                                hipStream_t s) {
    if (ncls <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_route_compact, dim3(ncls), dim3(1024), 0, s, cls, tmpl, prec, gate_val, slots,
                       live);
    return hipGetLastError();
}

hipError_t launch_newton_init(bool fp64, const FactorJob* jobs, int njobs, int ld,
                              const double* stats, void* scratch, const FactorDiag* diag,
                              const NewtonArgs& a, hipStream_t s) {
    if (njobs <= 0) return hipSuccess;
    // one workgroup per tile; factors up to 128 (chunks of the gated fp64
    // chain, where most factors exit at once) one workgroup per factor
    const dim3 grid(ld <= 128 ? 1 : (ld / 32) * (ld / 32), njobs);
    if (fp64)
        hipLaunchKernelGGL(k_newton_init<double>, grid, dim3(256), 0, s, jobs, stats,
                           static_cast<double*>(scratch), diag, a);
    else
        hipLaunchKernelGGL(k_newton_init<float>, grid, dim3(256), 0, s, jobs, stats,
                           static_cast<float*>(scratch), diag, a);
    return hipGetLastError();
}
hipError_t launch_newton_commit(bool fp64, const FactorJob* jobs, int njobs, int ld, float* arena,
                                const void* scratch, const void* scratch_m, FactorDiag* diag,
                                const NewtonArgs& a, hipStream_t s) {
    if (njobs <= 0) return hipSuccess;
    // one workgroup per tile; factors up to 128 (chunks of the gated fp64
    // chain, where most factors exit at once) one workgroup per factor
    const dim3 grid(ld <= 128 ? 1 : (ld / 32) * (ld / 32), njobs);
    if (fp64) {
        hipLaunchKernelGGL(k_newton_check<double>, grid, dim3(256), 0, s, jobs,
                           static_cast<const double*>(scratch), static_cast<const double*>(scratch_m),
                           diag, a);
        hipLaunchKernelGGL(k_newton_commit<double>, grid, dim3(256), 0, s, jobs, arena,
                           static_cast<const double*>(scratch), diag, a);
    } else {
        hipLaunchKernelGGL(k_newton_check<float>, grid, dim3(256), 0, s, jobs,
                           static_cast<const float*>(scratch), static_cast<const float*>(scratch_m),
                           diag, a);
        hipLaunchKernelGGL(k_newton_commit<float>, grid, dim3(256), 0, s, jobs, arena,
                           static_cast<const float*>(scratch), diag, a);
    }
    return hipGetLastError();
}
hipError_t launch_newton128(const FactorJob* jobs, int njobs, const double* stats, float* arena,
                            FactorDiag* diag, int32_t* prec, const FusedArgs& a, hipStream_t s) {
    if (njobs <= 0) return hipSuccess;
    switch (a.p) {
        case 1: hipLaunchKernelGGL(k_newton128<1>, dim3(njobs), dim3(256), 0, s, jobs, stats, arena, diag, prec, a); break;
        case 2: hipLaunchKernelGGL(k_newton128<2>, dim3(njobs), dim3(256), 0, s, jobs, stats, arena, diag, prec, a); break;
        case 4: hipLaunchKernelGGL(k_newton128<4>, dim3(njobs), dim3(256), 0, s, jobs, stats, arena, diag, prec, a); break;
        case 8: hipLaunchKernelGGL(k_newton128<8>, dim3(njobs), dim3(256), 0, s, jobs, stats, arena, diag, prec, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}
hipError_t launch_step128(const StepJob* jobs, int njobs, const RowChunk* fold, int nfold,
                          int n_tensors, const uint64_t* bases, float* arena, double alpha, double beta,
                          float delta, double* partA, double* partD, const UpdateArgs& ua,
                          hipStream_t s) {
    if (njobs <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_step128, dim3(njobs + nfold), dim3(1024), 0, s, jobs, njobs, fold, n_tensors,
                       bases, arena, alpha, beta, delta, partA, partD, ua);
    return hipGetLastError();
}
hipError_t launch_apply128(const ApplyJob* jobs, int njobs, const uint64_t* bases, float* arena,
                           float delta, double* partA, double* partD, const UpdateArgs& ua,
                           hipStream_t s) {
    if (njobs <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_apply128, dim3(njobs), dim3(512), 0, s, jobs, bases, arena, delta, partA,
                       partD, ua);
    return hipGetLastError();
}
hipError_t launch_copy_jobs(const CopyJob* jobs, int njobs, unsigned char* arena, hipStream_t s) {
    if (njobs <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_copy_jobs, dim3(njobs), dim3(256), 0, s, jobs, arena);
    return hipGetLastError();
}
hipError_t launch_sym_reduce(const SymReduceJob* jobs, const TileRef* tiles, int ntiles,
                             double* arena, double alpha, double beta, hipStream_t s) {
    if (ntiles <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_sym_reduce, dim3(ntiles), dim3(256), 0, s, jobs, tiles, arena, alpha, beta);
    return hipGetLastError();
}
hipError_t launch_sos_norm(const SosJob* jobs, int njobs, int nchunks, float* arena, float delta,
                           double* partA, hipStream_t s) {
    if (nchunks <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_sos_norm, dim3(nchunks), dim3(256), 0, s, jobs, njobs, arena, delta, partA);
    return hipGetLastError();
}
hipError_t launch_sos_update(const SosJob* jobs, int njobs, int nchunks, float* arena,
                             const float* scale, float lr, hipStream_t s) {
    if (nchunks <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_sos_update, dim3(nchunks), dim3(256), 0, s, jobs, njobs, arena, scale, lr);
    return hipGetLastError();
}
hipError_t launch_set_identity(const FactorJob* jobs, int njobs, float* arena, hipStream_t s) {
    if (njobs <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_set_identity, dim3(njobs), dim3(256), 0, s, jobs, arena);
    return hipGetLastError();
}
hipError_t launch_adagrad_norm(const BlockChunk* chunks, int nchunks, const uint64_t* bases,
                               float* arena, float delta, double* partA, hipStream_t s) {
    if (nchunks <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_adagrad_norm, dim3(nchunks), dim3(256), 0, s, chunks, bases, arena, delta,
                       partA);
    return hipGetLastError();
}
hipError_t launch_block_scale(const BlockNorms* bn, int nblocks, const double* partA,
                              const double* partD, float* scale, hipStream_t s) {
    if (nblocks <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_block_scale, dim3((nblocks + 3) / 4), dim3(256), 0, s, bn, nblocks,
                       partA, partD, scale);
    return hipGetLastError();
}
hipError_t launch_update(const RowChunk* chunks, int nchunks, const uint64_t* bases, int n_tensors,
                         float* arena, const float* scale, const UpdateArgs& a, hipStream_t s) {
    if (nchunks <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_update, dim3(nchunks), dim3(256), 0, s, chunks, bases, n_tensors, arena,
                       scale, a);
    return hipGetLastError();
}
hipError_t launch_sparse_rows(const SparseJob* jobs, int njobs, int64_t total, float* arena,
                              float lr, float delta, hipStream_t s) {
    if (njobs <= 0 || total <= 0) return hipSuccess;
    const int64_t nb = (total + 255) / 256;
    hipLaunchKernelGGL(k_sparse_rows, dim3((unsigned)nb), dim3(256), 0, s, jobs, njobs, total,
                       arena, lr, delta);
    return hipGetLastError();
}

}  // namespace shampoo
