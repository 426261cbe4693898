// C-ABI of libshampoo_mi355x.so: host planner, state layout and launch
// sequence of the Shampoo step ("Scalable Second Order Optimization for Deep
// Learning"; Shampoo-at-scale podcast transcript, cues 6-16).
//
// The planner splits every dense tensor into Lemma-2 blocks (cue 16), gives
// each block an L and an R factor, lays out one device state buffer owned by
// the caller, and precomputes every descriptor table the kernels read
// (batched-GEMM tasks and tile maps, Lanczos jobs, Newton jobs, elementwise
// row runs).  The per-call work is: refresh the gradient/weight pointer table
// when it changed, then enqueue the kernels on the caller's stream.
#include "../../include/shampoo.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <vector>

#include "common.hpp"
#include "kernels.hpp"

using namespace shampoo;

namespace {

constexpr int kTile = 128;            // batched-GEMM tile edge
constexpr int kFactorPad = 32;        // factor matrices padded to a multiple of this
constexpr int kXcds = 8;              // MI355X: 8 XCDs, workgroup b dispatched to XCD b % 8
constexpr int64_t kElemChunk = 16384; // elements per workgroup in elementwise kernels
constexpr int kRingSlots = 16;        // pinned staging slots for per-call tables
constexpr size_t kNewtonScratchBudget = size_t(4) << 30;  // bytes per precision (default)
constexpr int kSplitKTiles = 512;     // one-sided statistics: target tiles per launch
constexpr int kSplitKMin = 512;       // and shortest chunk of the long dimension
constexpr int kNewtonSplitTiles = 256;  // Newton stages with fewer tiles are split over k
constexpr int kPersistGrid = 512;       // workgroups of a persistent (packed, <= 128) fp64 stage
constexpr int kSosMaxChunks = 64;     // sparse one-sided tables: split-K chunks per call, at most,
constexpr int kSosMinRows = 256;      // of at least this many listed rows (measured best)

int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }
int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

struct TensorPlan {
    int64_t rows = 0, cols = 0;
    int kind = 0;
    int mode = 0;  // 0 Shampoo, 1 dense Adagrad, 2 sparse rows
    int64_t off_a = -1, off_mom = -1, off_d = -1;  // bytes
    bool fused = false;  // Shampoo tensor whose blocks are all <= 128: update inside the apply kernel
    int os_side = -1;    // one-sided (Lemma 1): 0 L (G G^T, D = P G), 1 R (G^T G, D = G P);
                         // a sparse-row table (mode 2) with os_side 1 gets its rows per call
    int first_block = 0, n_blocks = 0, nbc = 0;
};

struct BlockPlan {
    int tensor, r0, c0, mb, nb;
    int fl, fr;          // factor ids; a one-sided block has one factor (fl == fr)
    bool one_sided;      // the whole tensor, preconditioned on one side (Lemma 1)
    bool small;          // at most 128 x 128: fused statistics and apply kernels
    int64_t off_t;       // bytes: scratch T = G_b P_R (mb x nb)
    int d_slot, d_tiles; // ||D||^2 partial slots
    int a_slot, a_chunks;
};

struct FactorPlan {
    int block, side, dim, ld;
    int p = 4;                      // root exponent: P = (S + eps I)^(-1/p)
    int64_t off_s, off_p, off_p64;  // bytes (off_p64 = -1 when absent)
};

// A sparse-row table with one-sided preconditioning: what the per-call
// tables of its statistics and apply need.
struct SosPlan {
    int tensor, block, factor;
    int64_t part_off;    // split-K partials (bytes), kSosMaxChunks x ld^2 fp64
};

struct LaunchRef {
    int64_t tasks_off = 0, tiles_off = 0;  // bytes
    int ntiles = 0;
};

// One GEMM launch of a Newton iteration; a launch with few tiles is split
// over k into `parts` partial products that a second launch sums.
struct NewtonStage {
    LaunchRef gemm;
    bool sorted = false;   // tile table in slot order: the persistent GEMM form
    int chain = 1;         // products per slot run in order by one workgroup
    int parts = 1;
    int64_t sum_jobs_off = 0, sum_tiles_off = 0;   // SplitSumJob / TileRef tables (bytes)
    int sum_ntiles = 0;
};

struct NewtonChunk {
    int ld = 0;
    int p = 4;                               // root exponent of its factors
    int iters = 20;                          // coupled-Newton iterations (newton_iters_for)
    int njobs = 0;
    bool fused = false;                      // fp32, ld <= 128: one kernel, no scratch
    int64_t jobs_off = 0;                    // FactorJob table (bytes)
    bool compact = false;                    // gated fp64 chain on packed slots: the jobs
    int64_t slot_jobs_off = 0;               // are written on the device (arena bytes)
    std::vector<NewtonStage> stages[2];      // per parity
    std::vector<NewtonStage> first;          // iteration 0 (the start forms X_1)
    std::vector<NewtonStage> last[2];        // the last iteration: X T only (per parity)
};

// The launches of one root pass over a set of factors.
struct RootTables {
    int64_t lanczos_s_small_off = 0, lanczos_p_small_off = 0;   // factors with ld <= 128
    int64_t lanczos_s_big_off = 0, lanczos_p_big_off = 0;       // factors with ld > 128
    int n_lanczos_small = 0, n_lanczos_big = 0;
    int lanczos_big_max_n = 0;                                  // largest dimension above 128
    std::vector<NewtonChunk> chunks32, chunks64;
    std::vector<CompactClass> compact;       // classes of the packed fp64 chain
    int64_t compact_off = 0;
};

// Host-side table builder: tables are appended to one blob that is copied
// into the arena's table region at bind time.
struct Blob {
    std::vector<unsigned char> bytes;
    template <typename T>
    int64_t add(const std::vector<T>& v) {
        const int64_t off = align_up((int64_t)bytes.size(), 256);
        bytes.resize(off + v.size() * sizeof(T));
        if (!v.empty()) std::memcpy(bytes.data() + off, v.data(), v.size() * sizeof(T));
        return off;
    }
};

enum ProfCat : int {
    PC_STATS = 0, PC_LANCZOS_S, PC_LANCZOS_P, PC_NEWTON_INIT, PC_NEWTON_GEMM32, PC_NEWTON_GEMM64,
    PC_NEWTON_COMMIT, PC_ADAGRAD, PC_APPLY_T, PC_APPLY_D, PC_SCALE, PC_UPDATE, PC_SPARSE,
    PC_NEWTON_FUSED, PC_APPLY_FUSED, PC_STEP_FUSED, PC_STATS_SPLITK, PC_SOS_STATS, PC_SOS_NORM,
    PC_SOS_APPLY, PC_SOS_UPDATE, PC_ROUTE, PC_NEWTON_SPLIT, PC_STATS_SMALL,
    PC_COUNT
};
const char* const kProfNames[PC_COUNT] = {
    "stats_gram_f64", "lanczos_stats", "lanczos_roots", "newton_init", "newton_gemm_f32",
    "newton_gemm_f64", "newton_commit", "adagrad_norm", "apply_gemm_t", "apply_gemm_d",
    "block_scale", "update", "sparse_rows", "newton_fused_f32", "apply_fused", "step_fused",
    "stats_onesided", "stats_onesided_rows", "onesided_rows_norm", "apply_onesided_rows",
    "onesided_rows_update", "route_compact", "newton_split_sum", "stats_gram128"};

struct ProfRec {
    int cat;
    hipEvent_t a, b;
};

}  // namespace

struct shampoo_s {
    shampoo_config cfg{};
    int n = 0;
    std::vector<TensorPlan> tensors;
    std::vector<BlockPlan> blocks;
    std::vector<FactorPlan> factors;
    int n_sparse = 0;

    // arena layout (bytes)
    size_t total = 0;
    int64_t off_bases = 0, off_sparse = 0, off_tables = 0, off_diag = 0, off_prec = 0, off_chk = 0;
    int64_t off_lzwork = 0;
    int64_t off_slot_jobs = 0, off_slot_live = 0;  // packed fp64 chain: slot jobs and flags
    int64_t slot_tmpl_off = 0;                     // and the template job of every slot entry
    int64_t off_scr32 = 0, off_scr64 = 0, off_partA = 0, off_partD = 0, off_scale = 0;
    int64_t off_split32 = 0, off_split64 = 0;   // partial products of split Newton stages
    int n_partA = 0, n_partD = 0;
    Blob blob;  // static tables (offsets relative to off_tables)

    LaunchRef gram, apply1, apply2;   // blocks with a side > 128
    // the same products in split precision (apply_precision 1): T^T = P_R G^T
    // with the Adagrad pass of G fused in, then D = P_L T
    LaunchRef nt1, nt2;
    LaunchRef splitk;                 // one-sided statistics: partial products
    LaunchRef gsplit;                 // blocks > 128 when few: statistics split over k
    int64_t gred_jobs_off = 0, gred_tiles_off = 0;
    int n_gred_tiles = 0;             // and the fixed-order sum of their partials
    std::vector<SosPlan> sos;         // sparse-row tables with one-sided preconditioning
    int64_t off_sos_stats = 0, off_sos_apply = 0;  // their per-call tables
    int64_t symred_jobs_off = 0, symred_tiles_off = 0;
    int n_symred_tiles = 0;           // and their fixed-order sum
    int64_t apply128_off = 0;
    int n_apply128 = 0;               // blocks of at most 128 x 128
    int64_t step128_off = 0;          // the same blocks for the fused step kernel
    int64_t gram128_off = 0;
    int n_gram128 = 0;                // blocks of at most 128 x 128
    int64_t ident_jobs_off = 0;
    // root-pass tables: [0] every factor; [1 + q] part q of a staggered pass
    // (factors of the blocks b with b % root_parts == q)
    std::vector<RootTables> roots;
    // the allocation-free pass: every factor, batched-chain iterates in the
    // static device scratch (pointer-table entry 1 + 2n) in chunks that fit it
    RootTables roots_na;
    bool noalloc_ok = false;          // every chain slot fits the static scratch
    void* na_ptr = nullptr;           // this device's static scratch (set at bind)
    int device = -1;                  // the device current at bind
    // the asynchronous pass: per part, root tables on the snapshot/staging
    // areas and the copy jobs around them; a side stream and its events
    std::vector<RootTables> async_roots;
    std::vector<int64_t> async_begin_off, async_end_off;
    std::vector<int> async_begin_n, async_end_n;
    int64_t off_snap = 0, off_stage = 0;
    hipStream_t side = nullptr;
    hipEvent_t ev_fork = nullptr, ev_join = nullptr;
    // steps without a root pass: the statistics of the blocks above 128 on
    // this stream beside the apply (default priority)
    hipStream_t ovl = nullptr;
    hipEvent_t ov_fork = nullptr, ov_join = nullptr;
    int async_part = -1;             // part in flight, or -1
    int64_t blockchunks_off = 0, blocknorms_off = 0, rowchunks_off = 0;
    int n_blockchunks = 0, n_rowchunks = 0, n_blocknorms = 0;
    // steps through the fused kernel: its dense-Adagrad row chunks (larger,
    // for 1024 threads) and the update's remaining (Shampoo) chunks
    int64_t fold_off = 0, shampoo_rows_off = 0;
    int n_fold = 0, n_shampoo_rows = 0;
    std::vector<FactorDiag> diag_init;

    // binding
    unsigned char* arena = nullptr;
    bool bound = false;
    std::vector<uint64_t> bases_host;   // last uploaded pointer table
    bool bases_valid = false;
    unsigned char* ring = nullptr;      // pinned staging
    size_t slot_bytes = 0;
    hipEvent_t ring_ev[kRingSlots] = {};
    bool ring_used[kRingSlots] = {};
    int ring_next = 0;

    // optional per-kernel timing
    bool prof_on = false;
    std::vector<ProfRec> prof_pending;
    std::vector<hipEvent_t> prof_pool;
    int64_t prof_launches[PC_COUNT] = {};
    double prof_ms[PC_COUNT] = {};

    ~shampoo_s() {
        for (auto& r : prof_pending) {
            (void)hipEventDestroy(r.a);
            (void)hipEventDestroy(r.b);
        }
        for (auto e : prof_pool) (void)hipEventDestroy(e);
        for (int i = 0; i < kRingSlots; ++i)
            if (ring_ev[i]) (void)hipEventDestroy(ring_ev[i]);
        if (ring) (void)hipHostFree(ring);
        if (ev_fork) (void)hipEventDestroy(ev_fork);
        if (ev_join) (void)hipEventDestroy(ev_join);
        if (side) (void)hipStreamDestroy(side);
        if (ov_fork) (void)hipEventDestroy(ov_fork);
        if (ov_join) (void)hipEventDestroy(ov_join);
        if (ovl) (void)hipStreamDestroy(ovl);
    }
};

namespace {

bool use_fp32(const shampoo_config& c) { return c.root_mode != SHAMPOO_ROOT_F64; }
bool use_fp64(const shampoo_config& c) { return c.root_mode != SHAMPOO_ROOT_F32; }

int newton_stage_count(int p) {  // GEMM launches per iteration
    if (p == 1) return 1;
    int s = 1;                     // X T and T^2
    for (int q = 2; q < p; q *= 2) ++s;  // further squarings
    return s + 1;                  // M <- T^p M
}

// The tile entries of one task: all tiles, or a symmetric product's upper
// ones -- with trans bit 6 (fp64 statistics of at least four tiles per side)
// the tiles above the diagonal and then the groups of the diagonal band, four
// 64 x 64 units each, as tile indices -1 - q.
constexpr int kBandBit = 64;
void task_tiles(const GemmTask& t, int32_t i, std::vector<TileRef>& out) {
    const int nt = ceil_div(t.M, kTile) * t.tiles_n;
    const bool upper = (t.trans >> 4) & 1, band = t.trans & kBandBit;
    for (int e = 0; e < nt; ++e) {
        const int ti = e / t.tiles_n, tj = e % t.tiles_n;
        if (!upper || ti < tj || (ti == tj && !band)) out.push_back({i, e});
    }
    if (band)
        for (int q = 0; q < ceil_div(3 * t.tiles_n, 4); ++q) out.push_back({i, -1 - q});
}

// The band bit for a statistics task: the groups of four units cover the
// diagonal band of T tiles per side in ceil(3T / 4) workgroups instead of T.
int32_t band_bit(int tiles_n) { return tiles_n >= 4 ? kBandBit : 0; }

// The tile table of one batched-GEMM launch, in dispatch order.  Workgroup b
// runs on XCD b % 8, and each XCD has its own L2; the tiles of one task
// share its A and B panels.  So whole tasks go to XCDs (in order, each to the
// least-loaded one by tiles x K, which balances uneven tasks and spreads the
// tasks of a gated launch), the per-XCD counts are evened out by moving tail
// tiles, and the lists are interleaved: entry 8k + x is XCD x's k-th tile.
// `group` consecutive tasks that read the same operand (the L and R
// statistics of one block both read G_b) go to one XCD together, their tiles
// one after the other, so that the second task's reads can hit that L2.
std::vector<TileRef> xcd_tile_order(const std::vector<GemmTask>& tasks, int group = 1) {
    std::vector<std::vector<TileRef>> lists(kXcds);
    std::vector<double> load(kXcds, 0.0);
    size_t n = 0;
    const size_t gs = (size_t)std::max(group, 1);
    for (size_t i0 = 0; i0 < tasks.size(); i0 += gs) {
        const int x = (int)(std::min_element(load.begin(), load.end()) - load.begin());
        for (size_t i = i0; i < std::min(tasks.size(), i0 + gs); ++i) {
            const size_t before = lists[x].size();
            task_tiles(tasks[i], (int32_t)i, lists[x]);
            n += lists[x].size() - before;
            load[x] += (double)(lists[x].size() - before) * std::max(tasks[i].K, 1);
        }
    }
    const size_t q = n / kXcds, r = n % kXcds;
    std::vector<TileRef> pool;
    for (int x = 0; x < kXcds; ++x) {
        const size_t want = q + ((size_t)x < r ? 1 : 0);
        while (lists[x].size() > want) {
            pool.push_back(lists[x].back());
            lists[x].pop_back();
        }
    }
    for (int x = 0; x < kXcds; ++x) {
        const size_t want = q + ((size_t)x < r ? 1 : 0);
        while (lists[x].size() < want) {
            lists[x].push_back(pool.back());
            pool.pop_back();
        }
    }
    std::vector<TileRef> tiles;
    tiles.reserve(n);
    for (size_t k = 0; k <= q; ++k)
        for (int x = 0; x < kXcds; ++x)
            if (k < lists[x].size()) tiles.push_back(lists[x][k]);
    return tiles;
}

// A launch whose tile table is in task order (tasks sorted by gating id), for
// the persistent form of the GEMM kernel.
LaunchRef add_launch_sorted(Blob& blob, const std::vector<GemmTask>& tasks) {
    std::vector<TileRef> tiles;
    for (size_t i = 0; i < tasks.size(); ++i) task_tiles(tasks[i], (int32_t)i, tiles);
    LaunchRef L;
    L.tasks_off = blob.add(tasks);
    L.tiles_off = blob.add(tiles);
    L.ntiles = (int)tiles.size();
    return L;
}

LaunchRef add_launch(Blob& blob, const std::vector<GemmTask>& tasks, int group = 1) {
    const std::vector<TileRef> tiles = xcd_tile_order(tasks, group);
    LaunchRef L;
    L.tasks_off = blob.add(tasks);
    L.tiles_off = blob.add(tiles);
    L.ntiles = (int)tiles.size();
    return L;
}

// A launch of the split-precision C = A B^T kernel: its tiles in the same
// XCD-aware order as a batched-GEMM launch of the same shapes.
LaunchRef add_launch_nt(Blob& blob, const std::vector<NtTask>& tasks) {
    std::vector<GemmTask> shape(tasks.size());
    for (size_t i = 0; i < tasks.size(); ++i) {
        shape[i].M = tasks[i].M;
        shape[i].N = tasks[i].N;
        shape[i].K = tasks[i].K;
        shape[i].tiles_n = tasks[i].tiles_n;
    }
    const std::vector<TileRef> tiles = xcd_tile_order(shape);
    LaunchRef L;
    L.tasks_off = blob.add(tasks);
    L.tiles_off = blob.add(tiles);
    L.ntiles = (int)tiles.size();
    return L;
}

// Split-K parts for a Newton stage of `tiles` upper 128 x 128 tiles over
// k = ld: 1 when the stage already fills the GPU, else the largest power of
// two up to 8 that keeps the parts' tiles within 1024 and each part a
// multiple of 32 and at least 64 deep.
int newton_split(int tiles, int ld) {
    if (tiles >= kNewtonSplitTiles) return 1;
    int s = 1;
    while (s < 8 && tiles * s * 2 <= 1024 && ld % (64 * s) == 0 && ld / (2 * s) >= 64) s *= 2;
    return s;
}

// Partial-product scratch of the split stages of a chunk of nf factors
// (stage 0 has two products per factor, the others one).
int64_t newton_split_bytes(int nf, int ld, int64_t esz) {
    const int t1 = ceil_div(ld, kTile), ut = t1 * (t1 + 1) / 2;
    int64_t best = 0;
    for (int tasks : {2 * nf, nf}) {
        const int parts = newton_split(tasks * ut, ld);
        if (parts > 1) best = std::max(best, (int64_t)tasks * parts * ld * ld * esz);
    }
    return best;
}

// Coupled-Newton iterations for exponent p.  newton_iters is the count at
// p = 4.  In the first phase of the iteration the smallest scaled eigenvalue
// of M grows by g_p = ((p + 1) / p)^p per step (2.44 at p = 4, 2.25 at p = 2,
// 2 at p = 1), so a smaller exponent takes newton_iters log g_4 / log g_p
// steps to close the same gap (a one-sided factor takes p = root_p / 2).
int newton_iters_for(const shampoo_config& c, int p) {
    if (p >= 4) return c.newton_iters;
    const double g4 = 4.0 * std::log(5.0 / 4.0), gp = p * std::log((p + 1.0) / p);
    return (int)std::ceil(c.newton_iters * g4 / gp);
}

// Per-step scaling of the batched coupled-Newton iteration (with a
// convergence exit, newton_tol > 0).  Step k scales M_k by mu_k and X_k by
// mu_k^(1/p) before T = ((p+1) I - M) / p is formed, which keeps
// M_k = X_k^p A; so the products take T' = mu^(1/p) ((p+1) I - mu M) / p in
// place of T, and X <- X T', M <- T'^p M.  Every eigenvalue m of M follows the
// scalar map f(m) = m ((p+1-m)/p)^p after the scaling.  The spectrum of M_0 =
// z A lies in [lo, hi] with lo = (p+1)/2 eps_rel / (1 + eps_rel) (A's
// eigenvalues are at least eps) and hi = (p+1)/2 (1 + 1e-2) (a margin for the
// estimate of lambda_max), so the interval is carried through the map and mu_k
// chosen from it alone: the largest mu with mu hi <= 0.7 (p+1) (T' keeps the
// top of the spectrum away from 0, where fp32 rounding would be amplified)
// and f(mu lo) <= f(mu hi) (the bottom's image is the new lower end), until lo
// reaches 1/2, and 1 after that.  mu is the same for every factor (it
// depends on p and eps_rel only), and so is the step count: conv_steps is the
// first k at which the interval of M_k lies within tau of 1, plus `extra`
// steps (at most iters).
void newton_schedule(int p, double eps_rel, int iters, double tau, int extra,
                     std::vector<double>& mu, int& conv_steps) {
    auto f = [p](double m) { return m * std::pow((p + 1 - m) / p, p); };
    double lo = 0.5 * (p + 1) * eps_rel / (1.0 + eps_rel), hi = 0.5 * (p + 1) * 1.01;
    const double cap = 0.7 * (p + 1);
    mu.assign(iters, 1.0);
    conv_steps = iters;
    bool found = false;
    for (int k = 0; k < iters; ++k) {
        if (!found && std::max(1.0 - lo, hi - 1.0) <= tau) {
            conv_steps = std::min(iters, k + extra);
            found = true;
        }
        double m = 1.0;
        if (lo < 0.5) {
            double a = 1.0 / hi, b = cap / hi;
            if (f(b * lo) <= f(b * hi)) {
                m = b;
            } else {
                for (int it = 0; it < 100; ++it) {   // f(c lo) - f(c hi) grows with c
                    const double c = 0.5 * (a + b);
                    if (f(c * lo) < f(c * hi)) a = c;
                    else b = c;
                }
                m = std::max(a, 1.0);
            }
        }
        mu[k] = m;
        const double x = f(m * lo), y = f(m * hi);
        const double top = (m * lo <= 1.0 && 1.0 <= m * hi) ? 1.0 : std::max(x, y);
        lo = std::min(x, y);
        hi = top;
    }
}

// Builds the per-parity GEMM launches of one Newton chunk.
// gids: the gating id of each factor's products (default: the factor id).
// split_off_bytes: the partial-product scratch of split stages.
// base_idx: pointer-table entry the products' offsets are relative to (0:
// the state buffer; the allocation-free pass: its static scratch).
// allow_split: stages with few tiles may be split over k.
void build_newton_chunk(shampoo_s* h, NewtonChunk& ch, const std::vector<int>& fids, int ld,
                        bool fp64, bool fused, int64_t scratch_off_bytes, int p,
                        int64_t split_off_bytes, const std::vector<int>* gids = nullptr,
                        int base_idx = 0, bool allow_split = true) {
    ch.p = p;
    ch.iters = newton_iters_for(h->cfg, p);
    const int64_t esz = fp64 ? 8 : 4;
    const int64_t mat = (int64_t)ld * ld;
    const int64_t sbase = scratch_off_bytes / esz;  // scratch start in elements (arena base 0)
    const int tiles1 = ceil_div(ld, kTile);
    ch.ld = ld;
    ch.njobs = (int)fids.size();
    std::vector<FactorJob> jobs;
    for (size_t s = 0; s < fids.size(); ++s) {
        const FactorPlan& f = h->factors[fids[s]];
        FactorJob j{};
        j.s_off = f.off_s / 8;
        j.p_off = f.off_p / 4;
        j.p64_off = f.off_p64 >= 0 ? f.off_p64 / 8 : -1;
        j.x_off = (int64_t)s * 6 * mat;      // relative to the scratch pointer
        j.m_off = j.x_off + 2 * mat;
        j.n = f.dim;
        j.ld = ld;
        j.factor = fids[s];
        jobs.push_back(j);
    }
    ch.jobs_off = h->blob.add(jobs);
    ch.fused = fused;
    if (fused) return;

    auto mk = [&](int64_t a, int64_t b, int64_t c, int trans, int fid) {
        GemmTask t{};
        t.a_off = sbase + a; t.b_off = sbase + b; t.c_off = sbase + c;
        t.a_base = t.b_base = t.c_base = base_idx;
        t.M = t.N = t.K = ld;
        t.lda = t.ldb = t.ldc = ld;
        // a square of one symmetric operand (the same transform on both
        // sides) stages equal A and B panels: its diagonal band in groups
        const bool square = a == b && ((trans >> 2) & 1) == ((trans >> 3) & 1) && (trans & 16);
        t.trans = trans | (square ? band_bit(tiles1) : 0);
        t.tiles_n = tiles1;
        t.factor = fid;
        t.norm_slot = -1;
        return t;
    };
    // the launches of one iteration's stages (products per stage, per slot)
    auto emit = [&](const std::vector<std::vector<GemmTask>>& st, std::vector<NewtonStage>& out) {
        // a packed fp64 chain of factors up to 128 (one tile per product):
        // one launch per iteration in the persistent form, each workgroup
        // taking a slot's products in order (X T, T^2, ..., T^p M); with
        // nothing routed that is one launch of a few hundred workgroups that
        // stop at once, instead of one launch per stage and a workgroup per tile
        if (fp64 && gids != nullptr && ld <= kTile) {   // the persistent form is fp64 only
            const size_t n = fids.size();
            std::vector<GemmTask> seq;
            int per = 0;
            for (size_t k = 0; k < st.size(); ++k) per += (int)(st[k].size() / n);
            for (size_t sl = 0; sl < n; ++sl)
                for (size_t k = 0; k < st.size(); ++k) {
                    const size_t m = st[k].size() / n;   // products of this stage per slot
                    for (size_t j = 0; j < m; ++j) seq.push_back(st[k][sl * m + j]);
                }
            NewtonStage ns;
            ns.sorted = true;
            ns.chain = per;
            ns.gemm = add_launch_sorted(h->blob, seq);
            out.push_back(ns);
            return;
        }
        // a stage with few tiles is split over k: part c of a product sums
        // k in [c ld/parts, (c+1) ld/parts) into its own partial (upper
        // tiles), and the sum writes both triangles of the destination
        const int ut = tiles1 * (tiles1 + 1) / 2;
        for (auto& tasks : st) {
            NewtonStage ns;
            const int parts = allow_split ? newton_split((int)tasks.size() * ut, ld) : 1;
            if (parts == 1) {
                // the products of one slot in a stage (X T(M) and T(M)^2 both
                // read M) on one XCD
                const int per = fids.empty() ? 1 : (int)(tasks.size() / fids.size());
                ns.gemm = add_launch(h->blob, tasks, per);
            } else {
                const int64_t pbase = split_off_bytes / esz;
                const int kp = ld / parts, t32 = ld / 32;
                std::vector<GemmTask> sp;
                std::vector<SplitSumJob> jobs;
                std::vector<TileRef> tl;
                for (size_t i = 0; i < tasks.size(); ++i) {
                    const GemmTask& t = tasks[i];
                    const int64_t po = pbase + (int64_t)i * parts * mat;
                    for (int c = 0; c < parts; ++c) {
                        GemmTask u = t;
                        u.kb = c * kp;
                        u.K = (c + 1) * kp;
                        u.c_off = po + c * mat;
                        u.trans &= ~32;
                        sp.push_back(u);
                    }
                    jobs.push_back(SplitSumJob{po, t.c_off, parts, ld, t32, t.factor});
                    for (int bi = 0; bi < t32; ++bi)
                        for (int bj = bi; bj < t32; ++bj) tl.push_back(TileRef{(int32_t)i, bi * t32 + bj});
                }
                ns.gemm = add_launch(h->blob, sp);
                ns.parts = parts;
                ns.sum_jobs_off = h->blob.add(jobs);
                ns.sum_tiles_off = h->blob.add(tl);
                ns.sum_ntiles = (int)tl.size();
            }
            out.push_back(ns);
        }
    };
    for (int q = 0; q < 2; ++q) {
        std::vector<std::vector<GemmTask>> st(newton_stage_count(p));
        for (size_t s = 0; s < fids.size(); ++s) {
            const int64_t b = (int64_t)s * 6 * mat;
            const int64_t Xq = b + q * mat, Xn = b + (1 - q) * mat;
            const int64_t Mq = b + (2 + q) * mat, Mn = b + (3 - q) * mat;
            const int64_t T2 = b + 4 * mat, T4 = b + 5 * mat;
            const int fid = gids ? (*gids)[s] : fids[s];
            // stage 0: X <- X T(M) and T(M)^2 (p = 1: M <- T(M) M).  X, M and
            // T(M) are polynomials in the same matrix A, so every product
            // here is symmetric: upper tiles only (16), mirrored (32)
            st[0].push_back(mk(Xq, Mq, Xn, 8 | 16 | 32, fid));
            if (p == 1) {
                st[0].push_back(mk(Mq, Mq, Mn, 4 | 16 | 32, fid));
                continue;
            }
            // the squarings and the M update likewise
            st[0].push_back(mk(Mq, Mq, T2, 4 | 8 | 16 | 32, fid));
            int k = 1;
            int64_t cur = T2;
            for (int e = 2; e < p; e *= 2) {
                const int64_t nxt = (cur == T2) ? T4 : T2;
                st[k++].push_back(mk(cur, cur, nxt, 16 | 32, fid));
                cur = nxt;
            }
            st[k].push_back(mk(cur, Mq, Mn, 16 | 32, fid));
        }
        emit(st, ch.stages[q]);
        {
            // the last iteration's M is not needed: its X T products alone
            std::vector<std::vector<GemmTask>> stl(1);
            for (size_t i = 0; i < st[0].size(); i += 2) stl[0].push_back(st[0][i]);
            emit(stl, ch.last[q]);
        }
        if (q == 0) {
            // iteration 0 without X T: X_0 is diagonal, and the start writes
            // X_1 = X_0 T(M_0) itself (stage 0 holds X T and one more product
            // per slot)
            std::vector<std::vector<GemmTask>> st0 = st;
            st0[0].clear();
            for (size_t i = 1; i < st[0].size(); i += 2) st0[0].push_back(st[0][i]);
            emit(st0, ch.first);
        }
    }
}

int build_plan(shampoo_s* h) {
    const shampoo_config& c = h->cfg;
    const int b = c.block_size;
    int64_t off = 0;
    auto take = [&](int64_t bytes) {
        const int64_t o = align_up(off, 256);
        off = o + std::max<int64_t>(bytes, 0);
        return o;
    };

    // tensors and blocks
    for (int t = 0; t < h->n; ++t) {
        TensorPlan& tp = h->tensors[t];
        if (tp.kind == SHAMPOO_SPARSE_ROWS) {
            tp.mode = 2;
            h->n_sparse++;
            // Lemma 1 for an embedding table: the column side, when it fits
            if (c.large_layer == 1 && (c.max_precond_dim <= 0 || tp.cols <= c.max_precond_dim))
                tp.os_side = 1;
            continue;
        }
        const bool shampoo = c.max_precond_dim <= 0 ||
                             (tp.rows <= c.max_precond_dim && tp.cols <= c.max_precond_dim);
        tp.mode = shampoo ? 0 : 1;
        if (!shampoo) {
            // Lemma 1: precondition the side that fits, the other not at all
            if (c.large_layer == 1) {
                if (tp.cols <= c.max_precond_dim) tp.os_side = 1;
                else if (tp.rows <= c.max_precond_dim) tp.os_side = 0;
            }
            if (tp.os_side >= 0) tp.mode = 0;
            continue;
        }
        tp.first_block = (int)h->blocks.size();
        tp.nbc = ceil_div(tp.cols, b);
        for (int64_t r0 = 0; r0 < tp.rows; r0 += b)
            for (int64_t c0 = 0; c0 < tp.cols; c0 += b) {
                BlockPlan bp{};
                bp.tensor = t;
                bp.r0 = (int)r0;
                bp.c0 = (int)c0;
                bp.mb = (int)std::min<int64_t>(b, tp.rows - r0);
                bp.nb = (int)std::min<int64_t>(b, tp.cols - c0);
                bp.fl = 2 * (int)h->blocks.size();
                bp.fr = bp.fl + 1;
                bp.small = bp.mb <= 128 && bp.nb <= 128;
                h->blocks.push_back(bp);
            }
        tp.n_blocks = (int)h->blocks.size() - tp.first_block;
        tp.fused = true;
        for (int k = tp.first_block; k < (int)h->blocks.size(); ++k) tp.fused = tp.fused && h->blocks[k].small;
    }
    // one-sided tensors: one block each, numbered after every Shampoo block
    const int n_regular = (int)h->blocks.size();
    for (int t = 0; t < h->n; ++t) {
        TensorPlan& tp = h->tensors[t];
        if (tp.os_side < 0) continue;
        BlockPlan bp{};
        bp.tensor = t;
        bp.r0 = bp.c0 = 0;
        bp.mb = (int)tp.rows;
        bp.nb = (int)tp.cols;
        bp.fl = bp.fr = 2 * n_regular + ((int)h->blocks.size() - n_regular);
        bp.one_sided = true;
        bp.small = false;
        tp.first_block = (int)h->blocks.size();
        tp.n_blocks = 1;
        tp.nbc = 1;
        h->blocks.push_back(bp);
    }
    for (size_t i = 0; i < h->blocks.size(); ++i) {
        const BlockPlan& bp = h->blocks[i];
        for (int side = 0; side < 2; ++side) {
            const int os = h->tensors[bp.tensor].os_side;
            if (bp.one_sided && side != os) continue;
            FactorPlan f{};
            f.block = (int)i;
            f.side = side;
            f.dim = side == 0 ? bp.mb : bp.nb;
            f.ld = (int)align_up(f.dim, kFactorPad);
            f.p = bp.one_sided ? c.root_p / 2 : c.root_p;
            f.off_p64 = -1;
            h->factors.push_back(f);
        }
    }
    const int nf = (int)h->factors.size();
    const int nb = (int)h->blocks.size();

    // arena: per-call tables, diagnostics, factor matrices
    // pointer table: the state buffer, n gradients, n weights, the static
    // scratch of the allocation-free root pass
    h->off_bases = take((2 + 2 * (int64_t)h->n) * 8);
    h->off_sparse = take((int64_t)std::max(h->n_sparse, 1) * sizeof(SparseJob));
    h->off_diag = take((int64_t)std::max(nf, 1) * sizeof(FactorDiag));
    h->off_prec = take((int64_t)std::max(nf, 1) * 4);
    h->off_chk = take((int64_t)std::max(nf, 1) * 16);   // Newton finish: per-factor check slots
    h->off_lzwork = take((int64_t)kLanczosSplitMax * kLzWork * 8);  // split Lanczos records
    for (auto& f : h->factors) f.off_s = take((int64_t)f.ld * f.ld * 8);  // fp64 statistics
    for (auto& f : h->factors) f.off_p = take((int64_t)f.ld * f.ld * 4);
    if (use_fp64(c))
        for (auto& f : h->factors) f.off_p64 = take((int64_t)f.ld * f.ld * 8);

    // tensors: accumulators, momentum, preconditioned gradient
    for (auto& tp : h->tensors) {
        const int64_t numel = tp.rows * tp.cols;
        tp.off_a = take(numel * 4);
        if (tp.mode != 2) tp.off_mom = take(numel * 4);
        if ((tp.mode == 0 && !tp.fused) || (tp.mode == 2 && tp.os_side >= 0))
            tp.off_d = take(numel * 4);   // sparse one-sided: D of the listed rows
    }
    for (auto& bp : h->blocks)
        bp.off_t = (bp.small || bp.one_sided) ? -1 : take((int64_t)bp.mb * bp.nb * 4);
    // one-sided statistics: the product over the long dimension is split into
    // chunks (enough 128 x 128 tiles to fill the GPU); one fp64 partial per chunk
    std::vector<int> splitk_chunks(h->blocks.size(), 0), splitk_len(h->blocks.size(), 0);
    std::vector<int64_t> splitk_at(h->blocks.size(), -1);
    for (size_t i = 0; i < h->blocks.size(); ++i) {
        const BlockPlan& bp = h->blocks[i];
        if (!bp.one_sided) continue;
        const FactorPlan& f = h->factors[bp.fl];
        if (h->tensors[bp.tensor].mode == 2) {   // rows per call: chunks fixed per call
            splitk_at[i] = take((int64_t)kSosMaxChunks * f.ld * f.ld * 8);
            h->sos.push_back({bp.tensor, (int)i, bp.fl, splitk_at[i]});
            continue;
        }
        const int64_t K = f.side == 1 ? bp.mb : bp.nb;       // the long dimension
        const int ut = ceil_div(f.dim, kTile) * (ceil_div(f.dim, kTile) + 1) / 2;
        const int want = std::max(1, ceil_div(kSplitKTiles, ut));
        const int64_t len = align_up(std::max<int64_t>(ceil_div(K, want), kSplitKMin), 32);
        splitk_len[i] = (int)std::min<int64_t>(len, K);
        splitk_chunks[i] = ceil_div(K, splitk_len[i]);
        splitk_at[i] = take((int64_t)splitk_chunks[i] * f.ld * f.ld * 8);
    }
    // statistics of the blocks above 128: when all their upper 128 x 128 tiles
    // would leave most of the GPU idle (a few large blocks), each product is
    // split over k as well, into parts of at least 256 (multiples of 32)
    auto upper_tiles = [](int d) { const int t = ceil_div(d, kTile); return t * (t + 1) / 2; };
    int gram_tiles = 0;
    for (auto& bp : h->blocks)
        if (!bp.one_sided && !bp.small) gram_tiles += upper_tiles(bp.mb) + upper_tiles(bp.nb);
    const int gram_parts = (gram_tiles > 0 && gram_tiles < kNewtonSplitTiles)
                               ? std::min(8, ceil_div(2 * kNewtonSplitTiles, gram_tiles)) : 1;
    // per block: part length over the columns (L) and over the rows (R)
    std::vector<int> glen_l(h->blocks.size(), 0), glen_r(h->blocks.size(), 0);
    std::vector<int64_t> gsplit_at(h->blocks.size(), -1);
    if (gram_parts > 1)
        for (size_t i = 0; i < h->blocks.size(); ++i) {
            const BlockPlan& bp = h->blocks[i];
            if (bp.one_sided || bp.small) continue;
            auto len_of = [&](int K) {
                return (int)std::min<int64_t>(K, align_up(std::max(ceil_div(K, gram_parts), 256), 32));
            };
            glen_l[i] = len_of(bp.nb);
            glen_r[i] = len_of(bp.mb);
            const int64_t ldl = h->factors[bp.fl].ld, ldr = h->factors[bp.fr].ld;
            gsplit_at[i] = take((ceil_div(bp.nb, glen_l[i]) * ldl * ldl +
                                 ceil_div(bp.mb, glen_r[i]) * ldr * ldr) * 8);
        }

    // norm partial slots
    int na = 0, nd = 0;
    const bool split_apply = c.apply_precision == 1;
    for (auto& bp : h->blocks) {
        const int rows_per = (int)std::max<int64_t>(1, kElemChunk / bp.nb);
        bp.a_slot = na;
        // split-precision apply: the first product's tiles take the Adagrad
        // pass of the block between them, one partial per tile
        bp.a_chunks = bp.small ? 1
                      : (split_apply && !bp.one_sided) ? ceil_div(bp.nb, kTile) * ceil_div(bp.mb, kTile)
                                                        : ceil_div(bp.mb, rows_per);
        na += bp.a_chunks;
        bp.d_slot = nd;
        bp.d_tiles = bp.small ? 1 : ceil_div(bp.mb, kTile) * ceil_div(bp.nb, kTile);
        nd += bp.d_tiles;
    }
    h->n_partA = na;
    h->n_partD = nd;
    h->off_partA = take((int64_t)std::max(na, 1) * 8);
    h->off_partD = take((int64_t)std::max(nd, 1) * 8);
    h->off_scale = take((int64_t)std::max(nb, 1) * 4);

    // Newton root classes (by padded dimension) and scratch chunks
    std::vector<std::pair<int, int>> lds;   // (ld, p) classes
    for (auto& f : h->factors) lds.push_back({f.ld, f.p});
    std::sort(lds.begin(), lds.end());
    lds.erase(std::unique(lds.begin(), lds.end()), lds.end());
    int64_t scr32 = 0, scr64 = 0;
    struct Pending {
        int set; int ld; int p; std::vector<int> fids; bool fp64; bool fused;
        bool compact = false; int cap = 0; int slot_first = 0;
    };
    int n_slots = 0;
    std::map<std::pair<int, int>, int> na_slot_first;   // (ld, p) -> first slot, every factor
    int64_t split32 = 0, split64 = 0;
    int64_t scratch_budget = (int64_t)kNewtonScratchBudget;
    if (const char* e = std::getenv("SHAMPOO_NEWTON_SCRATCH_BYTES")) {
        const long long v = std::atoll(e);
        if (v > 0) scratch_budget = v;
    }
    std::vector<Pending> pend;
    // sets: 0 every factor; 1..P the parts of a staggered pass; P+1..2P the
    // same parts reading a snapshot of their statistics and writing staged
    // roots (the asynchronous pass on the library's own stream)
    const int nparts = c.root_parts > 1 ? c.root_parts : 0;
    h->roots.assign(1 + nparts, RootTables{});
    h->async_roots.assign(nparts, RootTables{});
    auto part_of = [&](int set) { return set <= nparts ? set - 1 : set - 1 - nparts; };
    auto in_set = [&](int set, int i) {
        return set == 0 || h->factors[i].block % nparts == part_of(set);
    };
    for (int set = 0; set <= 2 * nparts; ++set)
    for (auto [ld, pe] : lds) {
        std::vector<int> fids;
        for (int i = 0; i < nf; ++i)
            if (h->factors[i].ld == ld && h->factors[i].p == pe && in_set(set, i)) fids.push_back(i);
        if (fids.empty()) continue;
        for (int prec = 0; prec < 2; ++prec) {
            const bool fp64 = prec == 1;
            if ((fp64 && !use_fp64(c)) || (!fp64 && !use_fp32(c))) continue;
            if (!fp64 && ld <= 128) {   // fused LDS-resident kernel, no scratch
                pend.push_back(Pending{set, ld, pe, fids, false, true});
                continue;
            }
            const int64_t per = 6 * (int64_t)ld * ld * (fp64 ? 8 : 4);
            const int cap = (int)std::max<int64_t>(1, scratch_budget / per);
            if (fp64 && c.root_mode == SHAMPOO_ROOT_AUTO) {
                // the gated fp64 chain of AUTO runs on packed slots: the
                // routed factors of the class fill its first chunks
                Pending pd{set, ld, pe, fids, true, false};
                pd.compact = true;
                pd.cap = cap;
                pd.slot_first = n_slots;
                if (set == 0) na_slot_first[{ld, pe}] = n_slots;
                n_slots += (int)fids.size();
                const int n = (int)fids.size();
                scr64 = std::max(scr64, per * (int64_t)std::min(n, cap));
                // chunks of cap slots and a last, smaller one (factors up to
                // 128 run their products per slot, never split)
                if (ld > kTile) {
                    split64 = std::max(split64, newton_split_bytes(std::min(n, cap), ld, 8));
                    if (n > cap && n % cap) split64 = std::max(split64, newton_split_bytes(n % cap, ld, 8));
                }
                pend.push_back(std::move(pd));
                continue;
            }
            for (size_t s = 0; s < fids.size(); s += cap) {
                Pending pd;
                pd.set = set;
                pd.ld = ld;
                pd.p = pe;
                pd.fp64 = fp64;
                pd.fused = false;
                pd.fids.assign(fids.begin() + s, fids.begin() + std::min(fids.size(), s + cap));
                int64_t& scr = fp64 ? scr64 : scr32;
                scr = std::max(scr, per * (int64_t)pd.fids.size());
                int64_t& spl = fp64 ? split64 : split32;
                spl = std::max(spl, newton_split_bytes((int)pd.fids.size(), ld, fp64 ? 8 : 4));
                pend.push_back(std::move(pd));
            }
        }
    }
    h->off_scr32 = take(scr32);
    h->off_scr64 = take(scr64);
    h->off_split32 = take(split32);
    h->off_split64 = take(split64);
    h->off_slot_jobs = take((int64_t)n_slots * sizeof(FactorJob));
    h->off_slot_live = take((int64_t)n_slots * 4);
    // snapshot (fp64 statistics) and staging (fp32 roots) areas of the
    // asynchronous pass, sized for the largest part; per-factor places
    std::vector<int64_t> snap_at(nf, -1), stage_at(nf, -1);
    if (nparts > 0) {
        int64_t snap_max = 0, stage_max = 0;
        std::vector<int64_t> snap_rel(nf), stage_rel(nf);
        for (int q = 0; q < nparts; ++q) {
            int64_t a = 0, b = 0;
            for (int i = 0; i < nf; ++i) {
                if (h->factors[i].block % nparts != q) continue;
                const int64_t ld = h->factors[i].ld;
                snap_rel[i] = a;
                stage_rel[i] = b;
                a += ld * ld * 8;
                b += ld * ld * 4;
            }
            snap_max = std::max(snap_max, a);
            stage_max = std::max(stage_max, b);
        }
        h->off_snap = take(snap_max);
        h->off_stage = take(stage_max);
        for (int i = 0; i < nf; ++i) {
            snap_at[i] = h->off_snap + snap_rel[i];
            stage_at[i] = h->off_stage + stage_rel[i];
        }
    }
    // per-call tables of the sparse one-sided tables (largest possible call)
    if (!h->sos.empty()) {
        int64_t st = 0, ap = 0;
        const int64_t n = (int64_t)h->sos.size();
        for (const SosPlan& sp : h->sos) {
            const FactorPlan& f = h->factors[sp.factor];
            const BlockPlan& bp = h->blocks[sp.block];
            const int64_t t1 = ceil_div(f.dim, kTile), t32 = ceil_div(f.dim, 32);
            st += kSosMaxChunks * (int64_t)(sizeof(GemmTask) + t1 * (t1 + 1) / 2 * sizeof(TileRef)) +
                  t32 * (t32 + 1) / 2 * (int64_t)sizeof(TileRef);
            ap += (int64_t)ceil_div(bp.mb, kTile) * ceil_div(bp.nb, kTile) * sizeof(TileRef);
        }
        st += n * (int64_t)sizeof(SymReduceJob) + 4 * 256;
        ap += n * (int64_t)(sizeof(SosJob) + sizeof(GemmTask) + sizeof(BlockNorms)) + 4 * 256;
        h->off_sos_stats = take(st);
        h->off_sos_apply = take(ap);
    }
    h->off_tables = align_up(off, 256);

    // ---- static tables
    Blob& blob = h->blob;
    // statistics: L = beta2 L + w G G^T, R = beta2 R + w G^T G (cue 10).
    // Blocks of at most 128 x 128 go to the fused kernel, larger ones to the
    // batched GEMM (two tasks per block).
    {
        // The statistics keep their upper triangle; the split Lanczos of a
        // pass with at most kLanczosSplitMax factors above 128 reads whole
        // rows, so only then are the off-diagonal tiles also stored mirrored.
        bool mirror_stats = false;
        {
            const int np = c.root_parts > 1 ? c.root_parts : 0;
            for (int set = 0; set <= np; ++set) {
                int nbig = 0;
                for (const FactorPlan& f : h->factors)
                    if (f.ld > 128 && (set == 0 || f.block % np == set - 1)) ++nbig;
                if (nbig > 0 && nbig <= kLanczosSplitMax) mirror_stats = true;
            }
        }
        const int mbit = mirror_stats ? 32 : 0;
        std::vector<GemmTask> tasks;
        std::vector<GramJob> small;
        std::vector<GemmTask> sk, gs;
        std::vector<SymReduceJob> red, gred;
        std::vector<TileRef> red_tiles, gred_tiles;
        for (size_t bi = 0; bi < h->blocks.size(); ++bi) {
            const BlockPlan& bp = h->blocks[bi];
            const TensorPlan& tp = h->tensors[bp.tensor];
            const FactorPlan& fl = h->factors[bp.fl];
            const FactorPlan& fr = h->factors[bp.fr];
            if (bp.one_sided && tp.mode == 2) continue;   // sparse rows: per call
            if (bp.one_sided) {
                // partial c: S_c = G_c^T G_c (R; G_c rows [c len, (c+1) len)) or
                // G_c G_c^T (L; G_c those columns), upper 128 x 128 tiles
                const FactorPlan& f = fl;
                const int len = splitk_len[bi];
                const int64_t K = f.side == 1 ? bp.mb : bp.nb;
                for (int ck = 0; ck < splitk_chunks[bi]; ++ck) {
                    GemmTask t{};
                    const int64_t k0 = (int64_t)ck * len;
                    t.a_base = t.b_base = 1 + bp.tensor;
                    t.a_off = t.b_off = f.side == 1 ? k0 * tp.cols : k0;
                    t.lda = t.ldb = (int)tp.cols;
                    t.c_base = 0;
                    t.c_off = splitk_at[bi] / 8 + (int64_t)ck * f.ld * f.ld;
                    t.ldc = f.ld;
                    t.M = t.N = f.dim;
                    t.K = (int)std::min<int64_t>(len, K - k0);
                    t.tiles_n = ceil_div(t.N, kTile);
                    t.trans = (f.side == 1 ? 1 : 2) | 16 | band_bit(t.tiles_n);
                    t.factor = -1;
                    t.norm_slot = -1;
                    sk.push_back(t);
                }
                SymReduceJob r{};
                r.part_off = splitk_at[bi] / 8;
                r.s_off = f.off_s / 8;
                r.nparts = splitk_chunks[bi];
                r.dim = f.dim;
                r.ld = f.ld;
                r.tiles = ceil_div(f.dim, 32);
                for (int a = 0; a < r.tiles; ++a)
                    for (int b2 = a; b2 < r.tiles; ++b2)
                        red_tiles.push_back({(int32_t)red.size(), a * r.tiles + b2});
                red.push_back(r);
                continue;
            }
            if (bp.mb <= 128 && bp.nb <= 128) {
                GramJob j{};
                j.g_base = 1 + bp.tensor;
                j.g_off = (int64_t)bp.r0 * tp.cols + bp.c0;
                j.ldg = (int)tp.cols;
                j.mb = bp.mb;
                j.nb = bp.nb;
                j.l_off = fl.off_s / 8;
                j.r_off = fr.off_s / 8;
                j.ld_l = fl.ld;
                j.ld_r = fr.ld;
                small.push_back(j);
                continue;
            }
            if (gsplit_at[bi] >= 0) {
                // part c of L: G_c G_c^T over columns [c len, ...) of G_b; of R:
                // G_c^T G_c over rows [c len, ...); upper tiles into partials
                int64_t at = gsplit_at[bi] / 8;
                for (int side = 0; side < 2; ++side) {
                    const FactorPlan& f = side == 0 ? fl : fr;
                    const int K = side == 0 ? bp.nb : bp.mb, len = side == 0 ? glen_l[bi] : glen_r[bi];
                    const int parts = ceil_div(K, len);
                    for (int ck = 0; ck < parts; ++ck) {
                        GemmTask t{};
                        const int64_t k0 = (int64_t)ck * len;
                        t.a_base = t.b_base = 1 + bp.tensor;
                        t.a_off = t.b_off = (int64_t)bp.r0 * tp.cols + bp.c0 +
                                            (side == 0 ? k0 : k0 * tp.cols);
                        t.lda = t.ldb = (int)tp.cols;
                        t.c_base = 0;
                        t.c_off = at + (int64_t)ck * f.ld * f.ld;
                        t.ldc = f.ld;
                        t.M = t.N = f.dim;
                        t.K = (int)std::min<int64_t>(len, K - k0);
                        t.tiles_n = ceil_div(t.N, kTile);
                        t.trans = (side == 0 ? 2 : 1) | 16 | band_bit(t.tiles_n);
                        t.factor = -1;
                        t.norm_slot = -1;
                        gs.push_back(t);
                    }
                    SymReduceJob r{};
                    r.part_off = at;
                    r.s_off = f.off_s / 8;
                    r.nparts = parts;
                    r.dim = f.dim;
                    r.ld = f.ld;
                    r.tiles = ceil_div(f.dim, 32);
                    for (int a = 0; a < r.tiles; ++a)
                        for (int b2 = a; b2 < r.tiles; ++b2)
                            gred_tiles.push_back({(int32_t)gred.size(), a * r.tiles + b2});
                    gred.push_back(r);
                    at += (int64_t)parts * f.ld * f.ld;
                }
                continue;
            }
            GemmTask t{};
            t.a_base = t.b_base = 1 + bp.tensor;
            t.a_off = t.b_off = (int64_t)bp.r0 * tp.cols + bp.c0;
            t.lda = t.ldb = (int)tp.cols;
            t.c_base = 0;
            t.factor = -1;
            t.norm_slot = -1;
            // L: op(A) = G_b (mb x nb), op(B) = G_b^T
            t.c_off = fl.off_s / 8;
            t.ldc = fl.ld;
            t.M = t.N = bp.mb;
            t.K = bp.nb;
            t.tiles_n = ceil_div(t.N, kTile);
            // symmetric: upper tiles (mirrored for a split Lanczos)
            t.trans = 2 | 16 | mbit | band_bit(t.tiles_n);
            tasks.push_back(t);
            // R: op(A) = G_b^T (nb x mb), op(B) = G_b
            t.c_off = fr.off_s / 8;
            t.ldc = fr.ld;
            t.M = t.N = bp.nb;
            t.K = bp.mb;
            t.tiles_n = ceil_div(t.N, kTile);
            t.trans = 1 | 16 | mbit | band_bit(t.tiles_n);
            tasks.push_back(t);
        }
        h->gram = add_launch(blob, tasks, 2);   // L and R of a block on one XCD
        h->n_gram128 = (int)small.size();
        h->gram128_off = blob.add(small);
        h->splitk = add_launch(blob, sk);
        h->symred_jobs_off = blob.add(red);
        h->symred_tiles_off = blob.add(red_tiles);
        h->n_symred_tiles = (int)red_tiles.size();
        h->gsplit = add_launch(blob, gs);
        h->gred_jobs_off = blob.add(gred);
        h->gred_tiles_off = blob.add(gred_tiles);
        h->n_gred_tiles = (int)gred_tiles.size();
    }
    // apply: T = G_b P_R, then D = P_L T with ||D||^2 partials (cue 10)
    {
        std::vector<GemmTask> t1, t2;
        std::vector<NtTask> n1, n2;
        std::vector<ApplyJob> small;
        std::vector<StepJob> steps;
        for (auto& bp : h->blocks) {
            const TensorPlan& tp = h->tensors[bp.tensor];
            const FactorPlan& fl = h->factors[bp.fl];
            const FactorPlan& fr = h->factors[bp.fr];
            if (bp.one_sided && tp.mode == 2) continue;   // sparse rows: per call
            if (bp.one_sided && split_apply && fl.side == 1) {
                // D = G P in split precision: C = A B^T with B = P (symmetric)
                NtTask u{};
                u.a_base = 1 + bp.tensor; u.a_off = 0; u.lda = (int)tp.cols;
                u.b_base = 0; u.b_off = fl.off_p / 4; u.ldb = fl.ld;
                u.c_base = 0; u.c_off = tp.off_d / 4; u.ldc = (int)tp.cols;
                u.M = bp.mb; u.N = bp.nb; u.K = bp.nb;
                u.tiles_n = ceil_div(u.N, kTile);
                u.norm_slot = bp.d_slot;
                u.acc_off = -1;
                n2.push_back(u);
                continue;
            }
            if (bp.one_sided) {
                // D = G P (R) or P G (L), with ||D||^2 partials per tile
                GemmTask u{};
                if (fl.side == 1) {
                    u.a_base = 1 + bp.tensor; u.a_off = 0; u.lda = (int)tp.cols;
                    u.b_base = 0; u.b_off = fl.off_p / 4; u.ldb = fl.ld;
                    u.K = bp.nb;
                } else {
                    u.a_base = 0; u.a_off = fl.off_p / 4; u.lda = fl.ld;
                    u.b_base = 1 + bp.tensor; u.b_off = 0; u.ldb = (int)tp.cols;
                    u.K = bp.mb;
                }
                u.c_base = 0; u.c_off = tp.off_d / 4; u.ldc = (int)tp.cols;
                u.M = bp.mb; u.N = bp.nb;
                u.trans = 0;
                u.tiles_n = ceil_div(u.N, kTile);
                u.factor = -1;
                u.norm_slot = bp.d_slot;
                t2.push_back(u);
                continue;
            }
            if (bp.small) {
                ApplyJob j{};
                const int64_t o = (int64_t)bp.r0 * tp.cols + bp.c0;
                j.g_base = 1 + bp.tensor;
                j.g_off = o;
                j.a_off = tp.off_a / 4 + o;
                j.d_off = tp.fused ? -1 : tp.off_d / 4 + o;
                j.m_off = tp.off_mom / 4 + o;
                j.w_base = 1 + h->n + bp.tensor;
                j.fuse = tp.fused ? 1 : 0;
                j.pl_off = fl.off_p / 4;
                j.pr_off = fr.off_p / 4;
                j.ldg = (int)tp.cols;
                j.mb = bp.mb;
                j.nb = bp.nb;
                j.ld_l = fl.ld;
                j.ld_r = fr.ld;
                j.slot_a = bp.a_slot;
                j.slot_d = bp.d_slot;
                small.push_back(j);
                StepJob sj{};
                sj.ap = j;
                sj.l_off = fl.off_s / 8;
                sj.r_off = fr.off_s / 8;
                steps.push_back(sj);
                continue;
            }
            if (split_apply) {
                // T^T = P_R G_b^T (nb x mb, at off_t): C = A B^T with A = P_R
                // and B = G_b, both k-contiguous; its tiles also run the
                // block's Adagrad pass.  Then D = P_L T: A = P_L and
                // B = T^T, whose rows are T's columns.
                NtTask t{};
                t.a_base = 0; t.a_off = fr.off_p / 4; t.lda = fr.ld;
                t.b_base = 1 + bp.tensor; t.b_off = (int64_t)bp.r0 * tp.cols + bp.c0;
                t.ldb = (int)tp.cols;
                t.c_base = 0; t.c_off = bp.off_t / 4; t.ldc = bp.mb;
                t.M = bp.nb; t.N = bp.mb; t.K = bp.nb;
                t.tiles_n = ceil_div(t.N, kTile);
                t.norm_slot = -1;
                t.acc_off = tp.off_a / 4 + (int64_t)bp.r0 * tp.cols + bp.c0;
                t.acc_slot = bp.a_slot;
                n1.push_back(t);
                NtTask u{};
                u.a_base = 0; u.a_off = fl.off_p / 4; u.lda = fl.ld;
                u.b_base = 0; u.b_off = bp.off_t / 4; u.ldb = bp.mb;
                u.c_base = 0; u.c_off = tp.off_d / 4 + (int64_t)bp.r0 * tp.cols + bp.c0;
                u.ldc = (int)tp.cols;
                u.M = bp.mb; u.N = bp.nb; u.K = bp.mb;
                u.tiles_n = ceil_div(u.N, kTile);
                u.norm_slot = bp.d_slot;
                u.acc_off = -1;
                n2.push_back(u);
                continue;
            }
            GemmTask t{};
            t.a_base = 1 + bp.tensor;
            t.a_off = (int64_t)bp.r0 * tp.cols + bp.c0;
            t.lda = (int)tp.cols;
            t.b_base = 0;
            t.b_off = fr.off_p / 4;
            t.ldb = fr.ld;
            t.c_base = 0;
            t.c_off = bp.off_t / 4;
            t.ldc = bp.nb;
            t.M = bp.mb; t.N = bp.nb; t.K = bp.nb;
            t.trans = 0;
            t.tiles_n = ceil_div(t.N, kTile);
            t.factor = -1;
            t.norm_slot = -1;
            t1.push_back(t);
            GemmTask u{};
            u.a_base = 0; u.a_off = fl.off_p / 4; u.lda = fl.ld;
            u.b_base = 0; u.b_off = bp.off_t / 4; u.ldb = bp.nb;
            u.c_base = 0; u.c_off = tp.off_d / 4 + (int64_t)bp.r0 * tp.cols + bp.c0;
            u.ldc = (int)tp.cols;
            u.M = bp.mb; u.N = bp.nb; u.K = bp.mb;
            u.trans = 0;
            u.tiles_n = ceil_div(u.N, kTile);
            u.factor = -1;
            u.norm_slot = bp.d_slot;
            t2.push_back(u);
        }
        h->apply1 = add_launch(blob, t1);
        h->apply2 = add_launch(blob, t2);
        h->nt1 = add_launch_nt(blob, n1);
        h->nt2 = add_launch_nt(blob, n2);
        h->n_apply128 = (int)small.size();
        h->apply128_off = blob.add(small);
        h->step128_off = blob.add(steps);
    }
    // Lanczos jobs on statistics and on roots; identity jobs
    {
        std::vector<LanczosJob> js, jp;
        std::vector<FactorJob> ident;
        for (int i = 0; i < nf; ++i) {
            const FactorPlan& f = h->factors[i];
            js.push_back({f.off_s / 8, f.dim, f.ld, i, f.p});
            jp.push_back({f.off_p / 4, f.dim, f.ld, i, f.p});
            FactorJob j{};
            j.p_off = f.off_p / 4;
            j.p64_off = f.off_p64 >= 0 ? f.off_p64 / 8 : -1;
            j.n = f.dim;
            j.ld = f.ld;
            j.factor = i;
            ident.push_back(j);
            FactorDiag d{};
            d.block = f.block;
            d.side = f.side;
            d.dim = f.dim;
            h->diag_init.push_back(d);
        }
        for (int set = 0; set <= 2 * nparts; ++set) {
            std::vector<LanczosJob> jss, jps, jsb, jpb;
            int max_n = 0;
            const bool async = set > nparts;
            for (int i = 0; i < nf; ++i) {
                if (!in_set(set, i)) continue;
                const bool big = h->factors[i].ld > 128;
                LanczosJob a = js[i], b = jp[i];
                if (async) {
                    a.off = snap_at[i] / 8;
                    b.off = stage_at[i] / 4;
                }
                (big ? jsb : jss).push_back(a);
                (big ? jpb : jps).push_back(b);
                if (big) max_n = std::max(max_n, h->factors[i].dim);
            }
            RootTables& rt = async ? h->async_roots[set - 1 - nparts] : h->roots[set];
            rt.lanczos_big_max_n = max_n;
            rt.n_lanczos_small = (int)jss.size();
            rt.n_lanczos_big = (int)jsb.size();
            rt.lanczos_s_small_off = blob.add(jss);
            rt.lanczos_p_small_off = blob.add(jps);
            rt.lanczos_s_big_off = blob.add(jsb);
            rt.lanczos_p_big_off = blob.add(jpb);
        }
        h->ident_jobs_off = blob.add(ident);
    }
    std::vector<FactorJob> slot_tmpl(n_slots);
    for (auto& pd : pend) {
        const bool async = pd.set > nparts;
        std::vector<std::pair<int64_t, int64_t>> saved;
        if (async)   // the job tables of this chunk read the snapshot, write the staging area
            for (int i : pd.fids) {
                saved.push_back({h->factors[i].off_s, h->factors[i].off_p});
                h->factors[i].off_s = snap_at[i];
                h->factors[i].off_p = stage_at[i];
            }
        RootTables& rt = async ? h->async_roots[pd.set - 1 - nparts] : h->roots[pd.set];
        const int64_t scr = pd.fp64 ? h->off_scr64 : h->off_scr32;
        if (pd.compact) {
            // template jobs of the class (scratch places are set when packed)
            const int n = (int)pd.fids.size();
            for (int k = 0; k < n; ++k) {
                const FactorPlan& f = h->factors[pd.fids[k]];
                FactorJob j{};
                j.s_off = f.off_s / 8;
                j.p_off = f.off_p / 4;
                j.p64_off = f.off_p64 >= 0 ? f.off_p64 / 8 : -1;
                j.n = f.dim;
                j.ld = pd.ld;
                j.factor = pd.fids[k];
                slot_tmpl[pd.slot_first + k] = j;
            }
            rt.compact.push_back(CompactClass{pd.slot_first, n, pd.cap, 0, (int64_t)pd.ld * pd.ld});
            // chunk q holds slots [q cap, (q+1) cap); its products are gated
            // by the slot flags
            for (int q0 = 0; q0 < n; q0 += pd.cap) {
                const int m = std::min(pd.cap, n - q0);
                std::vector<int> fids(pd.fids.begin() + q0, pd.fids.begin() + q0 + m), gids(m);
                for (int k = 0; k < m; ++k) gids[k] = pd.slot_first + q0 + k;
                NewtonChunk ch;
                build_newton_chunk(h, ch, fids, pd.ld, true, false, scr, pd.p, h->off_split64, &gids);
                ch.compact = true;
                ch.slot_jobs_off = h->off_slot_jobs + (int64_t)(pd.slot_first + q0) * sizeof(FactorJob);
                rt.chunks64.push_back(std::move(ch));
            }
        } else {
            NewtonChunk ch;
            build_newton_chunk(h, ch, pd.fids, pd.ld, pd.fp64, pd.fused, scr, pd.p,
                               pd.fp64 ? h->off_split64 : h->off_split32);
            (pd.fp64 ? rt.chunks64 : rt.chunks32).push_back(std::move(ch));
        }
        if (async)
            for (size_t k = 0; k < pd.fids.size(); ++k) {
                h->factors[pd.fids[k]].off_s = saved[k].first;
                h->factors[pd.fids[k]].off_p = saved[k].second;
            }
    }
    h->slot_tmpl_off = blob.add(slot_tmpl);
    for (auto& rt : h->roots) rt.compact_off = blob.add(rt.compact);
    for (auto& rt : h->async_roots) rt.compact_off = blob.add(rt.compact);
    // The allocation-free pass over every factor: the same Lanczos tables,
    // fused roots and packed-slot arrangement as the whole pass, its
    // batched-chain iterates in the static device scratch in chunks that fit
    // it, and no split stages (their partials would need more scratch).  The
    // fp32 chain, then the fp64 one, run in stream order, so both start at
    // the scratch's beginning; nothing in it needs clearing first (the start
    // writes every iterate a product reads, and products skip unrouted slots).
    {
        RootTables& na = h->roots_na;
        const RootTables& r0 = h->roots[0];
        na.lanczos_s_small_off = r0.lanczos_s_small_off;
        na.lanczos_p_small_off = r0.lanczos_p_small_off;
        na.lanczos_s_big_off = r0.lanczos_s_big_off;
        na.lanczos_p_big_off = r0.lanczos_p_big_off;
        na.n_lanczos_small = r0.n_lanczos_small;
        na.n_lanczos_big = r0.n_lanczos_big;
        na.lanczos_big_max_n = r0.lanczos_big_max_n;
        h->noalloc_ok = true;
        const int na_base = 1 + 2 * h->n;
        for (auto [ld, pe] : lds) {
            std::vector<int> fids;
            for (int i = 0; i < nf; ++i)
                if (h->factors[i].ld == ld && h->factors[i].p == pe) fids.push_back(i);
            if (fids.empty()) continue;
            for (int prec = 0; prec < 2; ++prec) {
                const bool fp64 = prec == 1;
                if ((fp64 && !use_fp64(c)) || (!fp64 && !use_fp32(c))) continue;
                if (!fp64 && ld <= 128) {
                    NewtonChunk ch;
                    build_newton_chunk(h, ch, fids, ld, false, true, 0, pe, 0);
                    na.chunks32.push_back(std::move(ch));
                    continue;
                }
                const int64_t per = 6 * (int64_t)ld * ld * (fp64 ? 8 : 4);
                if (per > (int64_t)kNoallocScratchBytes) {
                    h->noalloc_ok = false;
                    continue;
                }
                const int cap = (int)((int64_t)kNoallocScratchBytes / per);
                const int n = (int)fids.size();
                if (fp64 && c.root_mode == SHAMPOO_ROOT_AUTO) {
                    const int first = na_slot_first.at({ld, pe});
                    na.compact.push_back(CompactClass{first, n, cap, 0, (int64_t)ld * ld});
                    for (int q0 = 0; q0 < n; q0 += cap) {
                        const int m = std::min(cap, n - q0);
                        std::vector<int> sub(fids.begin() + q0, fids.begin() + q0 + m), gids(m);
                        for (int k = 0; k < m; ++k) gids[k] = first + q0 + k;
                        NewtonChunk ch;
                        build_newton_chunk(h, ch, sub, ld, true, false, 0, pe, 0, &gids, na_base,
                                           false);
                        ch.compact = true;
                        ch.slot_jobs_off = h->off_slot_jobs + (int64_t)(first + q0) * sizeof(FactorJob);
                        na.chunks64.push_back(std::move(ch));
                    }
                    continue;
                }
                for (int q0 = 0; q0 < n; q0 += cap) {
                    std::vector<int> sub(fids.begin() + q0, fids.begin() + std::min(n, q0 + cap));
                    NewtonChunk ch;
                    build_newton_chunk(h, ch, sub, ld, fp64, false, 0, pe, 0, nullptr, na_base, false);
                    (fp64 ? na.chunks64 : na.chunks32).push_back(std::move(ch));
                }
            }
        }
        na.compact_off = blob.add(na.compact);
    }
    // copy jobs of the asynchronous pass: snapshot S and P of a part, and the
    // swap of its staged roots
    h->async_begin_off.assign(nparts, 0);
    h->async_end_off.assign(nparts, 0);
    h->async_begin_n.assign(nparts, 0);
    h->async_end_n.assign(nparts, 0);
    for (int q = 0; q < nparts; ++q) {
        std::vector<CopyJob> b, e;
        for (int i = 0; i < nf; ++i) {
            const FactorPlan& f = h->factors[i];
            if (f.block % nparts != q) continue;
            const int64_t n2 = (int64_t)f.ld * f.ld;
            b.push_back({f.off_s, snap_at[i], n2 * 8});
            b.push_back({f.off_p, stage_at[i], n2 * 4});
            e.push_back({stage_at[i], f.off_p, n2 * 4});
        }
        h->async_begin_n[q] = (int)b.size();
        h->async_end_n[q] = (int)e.size();
        h->async_begin_off[q] = blob.add(b);
        h->async_end_off[q] = blob.add(e);
    }
    // elementwise tables
    {
        std::vector<BlockChunk> bcs;
        std::vector<BlockNorms> bns;
        for (size_t i = 0; i < h->blocks.size(); ++i) {
            const BlockPlan& bp = h->blocks[i];
            const TensorPlan& tp = h->tensors[bp.tensor];
            const int rows_per = (int)std::max<int64_t>(1, kElemChunk / bp.nb);
            if (tp.mode == 2) continue;   // sparse one-sided table: norms per call
            const bool fused_adagrad = c.apply_precision == 1 && !bp.small && !bp.one_sided;
            for (int k = 0; !bp.small && !fused_adagrad && k < bp.a_chunks; ++k) {
                BlockChunk q{};
                q.tensor = bp.tensor;
                q.block = (int)i;
                q.row0 = bp.r0 + k * rows_per;
                q.nrows = std::min(rows_per, bp.mb - k * rows_per);
                q.col0 = bp.c0;
                q.ncols = bp.nb;
                q.cols = (int)tp.cols;
                q.slot = bp.a_slot + k;
                q.a_off = tp.off_a / 4;
                bcs.push_back(q);
            }
            // a tensor whose blocks are all <= 128 is updated inside the fused
            // kernels, which form each block's graft scale themselves
            if (!tp.fused) bns.push_back({bp.a_slot, bp.a_chunks, bp.d_slot, bp.d_tiles, (int)i, 0});
        }
        h->n_blockchunks = (int)bcs.size();
        h->n_blocknorms = (int)bns.size();
        h->blockchunks_off = blob.add(bcs);
        h->blocknorms_off = blob.add(bns);
        std::vector<RowChunk> rcs;
        for (int t = 0; t < h->n; ++t) {
            const TensorPlan& tp = h->tensors[t];
            if (tp.mode == 2 || tp.fused) continue;
            const int rows_per = (int)std::max<int64_t>(1, kElemChunk / tp.cols);
            for (int64_t r0 = 0; r0 < tp.rows; r0 += rows_per) {
                RowChunk q{};
                q.tensor = t;
                q.mode = tp.mode;
                q.row0 = (int)r0;
                q.nrows = (int)std::min<int64_t>(rows_per, tp.rows - r0);
                q.cols = (int)tp.cols;
                q.block_size = tp.os_side >= 0 ? (1 << 30) : b;  // one-sided: one block
                q.first_block = tp.first_block;
                q.nbc = tp.nbc;
                q.a_off = tp.off_a / 4;
                q.m_off = tp.off_mom / 4;
                q.d_off = tp.mode == 0 ? tp.off_d / 4 : 0;
                rcs.push_back(q);
            }
        }
        h->n_rowchunks = (int)rcs.size();
        h->rowchunks_off = blob.add(rcs);
        std::vector<RowChunk> fold, rest;
        for (const RowChunk& q : rcs)
            if (q.mode == 0) rest.push_back(q);
        for (int t = 0; t < h->n; ++t) {
            const TensorPlan& tp = h->tensors[t];
            if (tp.mode != 1 || tp.fused) continue;
            const int rows_per = (int)std::max<int64_t>(1, 4 * kElemChunk / tp.cols);
            for (int64_t r0 = 0; r0 < tp.rows; r0 += rows_per) {
                RowChunk q{};
                q.tensor = t;
                q.mode = 1;
                q.row0 = (int)r0;
                q.nrows = (int)std::min<int64_t>(rows_per, tp.rows - r0);
                q.cols = (int)tp.cols;
                q.block_size = b;
                q.a_off = tp.off_a / 4;
                q.m_off = tp.off_mom / 4;
                fold.push_back(q);
            }
        }
        h->n_fold = (int)fold.size();
        h->fold_off = blob.add(fold);
        h->n_shampoo_rows = (int)rest.size();
        h->shampoo_rows_off = blob.add(rest);
    }
    h->total = (size_t)align_up(h->off_tables + (int64_t)blob.bytes.size(), 256);
    return SHAMPOO_OK;
}

int hip_err(hipError_t e) { return e == hipSuccess ? SHAMPOO_OK : SHAMPOO_E_HIP; }

hipEvent_t prof_event(shampoo_s* h) {
    if (!h->prof_pool.empty()) {
        hipEvent_t e = h->prof_pool.back();
        h->prof_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

// Brackets one kernel launch with two events when timing is enabled.
struct ProfScope {
    shampoo_s* h;
    int cat;
    hipStream_t s;
    hipEvent_t a = nullptr;
    ProfScope(shampoo_s* h_, int cat_, hipStream_t s_, bool active = true)
        : h(h_), cat(cat_), s(s_) {
        if (!h->prof_on || !active) return;
        a = prof_event(h);
        if (a && hipEventRecord(a, s) != hipSuccess) a = nullptr;
    }
    ~ProfScope() {
        if (!a) return;
        hipEvent_t b = prof_event(h);
        if (b && hipEventRecord(b, s) == hipSuccess) h->prof_pending.push_back({cat, a, b});
        else h->prof_pool.push_back(a);
    }
};

template <typename T>
T* at(shampoo_s* h, int64_t off_bytes) {
    return reinterpret_cast<T*>(h->arena + off_bytes);
}
template <typename T>
T* tab(shampoo_s* h, int64_t blob_off) {
    return reinterpret_cast<T*>(h->arena + h->off_tables + blob_off);
}

// Copies `bytes` of host data to the arena at `dst_off` through pinned
// staging slots (so the call stays asynchronous), one slot per piece.
int stage_upload(shampoo_s* h, const void* src, size_t bytes, int64_t dst_off, hipStream_t s) {
    while (bytes > h->slot_bytes) {
        const int rc = stage_upload(h, src, h->slot_bytes, dst_off, s);
        if (rc) return rc;
        src = static_cast<const unsigned char*>(src) + h->slot_bytes;
        dst_off += (int64_t)h->slot_bytes;
        bytes -= h->slot_bytes;
    }
    if (bytes == 0) return SHAMPOO_OK;
    const int k = h->ring_next;
    h->ring_next = (k + 1) % kRingSlots;
    if (h->ring_used[k]) {
        hipError_t e = hipEventSynchronize(h->ring_ev[k]);
        if (e != hipSuccess) return SHAMPOO_E_HIP;
    }
    unsigned char* slot = h->ring + (size_t)k * h->slot_bytes;
    std::memcpy(slot, src, bytes);
    hipError_t e = hipMemcpyAsync(h->arena + dst_off, slot, bytes, hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return SHAMPOO_E_HIP;
    e = hipEventRecord(h->ring_ev[k], s);
    if (e != hipSuccess) return SHAMPOO_E_HIP;
    h->ring_used[k] = true;
    return SHAMPOO_OK;
}

// The per-call pointer table: the state buffer, each tensor's gradient (for
// a sparse one-sided table, its row gradients) and weights.
int refresh_bases(shampoo_s* h, const float* const* grads, float* const* params,
                  const shampoo_sparse_rows* sparse, hipStream_t s) {
    std::vector<uint64_t> nb = h->bases_host;
    if (nb.empty()) nb.assign(2 + 2 * (size_t)h->n, 0);
    nb[0] = reinterpret_cast<uint64_t>(h->arena);
    nb[1 + 2 * h->n] = reinterpret_cast<uint64_t>(h->na_ptr);   // the static scratch
    for (int t = 0; t < h->n; ++t) {
        if (grads) nb[1 + t] = reinterpret_cast<uint64_t>(grads[t]);
        if (params) nb[1 + h->n + t] = reinterpret_cast<uint64_t>(params[t]);
    }
    if (sparse)
        for (const SosPlan& sp : h->sos)
            nb[1 + sp.tensor] = reinterpret_cast<uint64_t>(sparse[sp.tensor].row_grads);
    if (h->bases_valid && nb == h->bases_host) return SHAMPOO_OK;
    const int rc = stage_upload(h, nb.data(), nb.size() * 8, h->off_bases, s);
    if (rc != SHAMPOO_OK) return rc;
    h->bases_host = nb;
    h->bases_valid = true;
    return SHAMPOO_OK;
}

}  // namespace

// =================================================================== C-ABI
extern "C" {

int shampoo_create(const shampoo_config* cfg, int32_t n_tensors, const shampoo_tensor_desc* tensors,
                   shampoo_t** out) {
    if (!cfg || !tensors || !out || n_tensors < 1) return SHAMPOO_E_ARG;
    *out = nullptr;
    const shampoo_config& c = *cfg;
    if (c.block_size < 1 || c.newton_iters < 1 || c.max_precond_dim < 0 || c.lanczos_steps < 0)
        return SHAMPOO_E_ARG;
    if (!(c.beta2 > 0.0 && c.beta2 <= 1.0) || !(c.eps_rel >= 0.0) || !(c.graft_eps >= 0.0) ||
        !std::isfinite(c.beta1) || !std::isfinite(c.lr) || c.root_parts < 0 ||
        !(c.newton_tol >= 0.0 && c.newton_tol < 1.0))
        return SHAMPOO_E_ARG;
    if (c.root_mode < SHAMPOO_ROOT_F32 || c.root_mode > SHAMPOO_ROOT_AUTO) return SHAMPOO_E_ARG;
    if (c.root_p != 1 && c.root_p != 2 && c.root_p != 4 && c.root_p != 8)
        return SHAMPOO_E_UNSUPPORTED;
    if (c.large_layer != 0 && c.large_layer != 1) return SHAMPOO_E_ARG;
    if (c.apply_precision != 0 && c.apply_precision != 1) return SHAMPOO_E_ARG;
    // the split-precision apply multiplies by the roots, whose condition is
    // kappa(S + eps I)^(1/p): for p < 4 its rounding is amplified past the
    // fp32 apply's (p = 1 at kappa 1e6: about 1e-2 of the update)
    if (c.apply_precision == 1 && c.root_p < 4) return SHAMPOO_E_UNSUPPORTED;
    if (c.reserved != 0) return SHAMPOO_E_ARG;
    if (c.large_layer == 1 && c.root_p % 2) return SHAMPOO_E_UNSUPPORTED;  // exponent -2/root_p
    for (int t = 0; t < n_tensors; ++t) {
        const shampoo_tensor_desc& d = tensors[t];
        if (d.rows < 1 || d.cols < 1 || d.reserved != 0) return SHAMPOO_E_ARG;
        if (d.kind != SHAMPOO_DENSE && d.kind != SHAMPOO_SPARSE_ROWS) return SHAMPOO_E_ARG;
        if (d.rows > INT32_MAX || d.cols > (int64_t)1 << 20) return SHAMPOO_E_UNSUPPORTED;
    }
    shampoo_s* h = new (std::nothrow) shampoo_s();
    if (!h) return SHAMPOO_E_NOMEM;
    try {
        h->cfg = c;
        // lanczos_steps == 0: lambda_max by Lanczos until the top Ritz pair's
        // residual is within kLanczosTol of theta (checked after 12 steps,
        // every 4th to 32, every 8th after), at most 64 steps; 8 steps for
        // the kappa estimate
        h->n = n_tensors;
        h->tensors.resize(n_tensors);
        for (int t = 0; t < n_tensors; ++t) {
            h->tensors[t].rows = tensors[t].rows;
            h->tensors[t].cols = tensors[t].cols;
            h->tensors[t].kind = tensors[t].kind;
        }
        const int rc = build_plan(h);
        if (rc != SHAMPOO_OK) {
            delete h;
            return rc;
        }
        // factor dimensions above the Lanczos limit are not supported
        for (auto& f : h->factors)
            if (f.dim > 1024) {
                delete h;
                return SHAMPOO_E_UNSUPPORTED;
            }
    } catch (const std::bad_alloc&) {
        delete h;
        return SHAMPOO_E_NOMEM;
    }
    *out = h;
    return SHAMPOO_OK;
}

int shampoo_state_bytes(const shampoo_t* h, size_t* bytes) {
    if (!h || !bytes) return SHAMPOO_E_ARG;
    *bytes = h->total;
    return SHAMPOO_OK;
}

int shampoo_num_factors(const shampoo_t* h, int32_t* n_factors, int32_t* n_blocks) {
    if (!h) return SHAMPOO_E_ARG;
    if (n_factors) *n_factors = (int32_t)h->factors.size();
    if (n_blocks) *n_blocks = (int32_t)h->blocks.size();
    return SHAMPOO_OK;
}

int shampoo_block_info(const shampoo_t* h, int32_t block, shampoo_block_layout* out) {
    if (!h || !out || block < 0 || block >= (int32_t)h->blocks.size()) return SHAMPOO_E_ARG;
    const BlockPlan& bp = h->blocks[block];
    const FactorPlan& fl = h->factors[bp.fl];
    const FactorPlan& fr = h->factors[bp.fr];
    out->tensor = bp.tensor;
    out->one_sided = bp.one_sided ? 1 : 0;
    out->row0 = bp.r0;
    out->col0 = bp.c0;
    out->rows = bp.mb;
    out->cols = bp.nb;
    out->ld_l = fl.ld;
    out->ld_r = fr.ld;
    out->factor_l = bp.fl;
    out->factor_r = bp.fr;
    out->off_l = fl.off_s;
    out->off_r = fr.off_s;
    out->off_pl = fl.off_p;
    out->off_pr = fr.off_p;
    out->off_pl64 = fl.off_p64;
    out->off_pr64 = fr.off_p64;
    if (bp.one_sided) {   // only the side that was kept
        const bool r = fl.side == 1;
        (r ? out->ld_l : out->ld_r) = 0;
        (r ? out->factor_l : out->factor_r) = -1;
        (r ? out->off_l : out->off_r) = -1;
        (r ? out->off_pl : out->off_pr) = -1;
        (r ? out->off_pl64 : out->off_pr64) = -1;
    }
    return SHAMPOO_OK;
}

int shampoo_tensor_info(const shampoo_t* h, int32_t tensor, int64_t* adagrad_off, int64_t* mom_off,
                        int32_t* first_block, int32_t* n_blocks) {
    if (!h || tensor < 0 || tensor >= h->n) return SHAMPOO_E_ARG;
    const TensorPlan& tp = h->tensors[tensor];
    if (adagrad_off) *adagrad_off = tp.off_a;
    if (mom_off) *mom_off = tp.off_mom;
    if (first_block) *first_block = tp.first_block;
    if (n_blocks) *n_blocks = tp.n_blocks;
    return SHAMPOO_OK;
}

int shampoo_bind_state(shampoo_t* h, void* dev_state, size_t bytes, void* stream) {
    if (!h || !dev_state) return SHAMPOO_E_ARG;
    if ((reinterpret_cast<uintptr_t>(dev_state) & 255) != 0) return SHAMPOO_E_ARG;
    if (bytes < h->total) return SHAMPOO_E_STATE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    h->arena = static_cast<unsigned char*>(dev_state);
    h->bound = false;
    h->bases_valid = false;
    h->bases_host.clear();
    if (!h->ring) {
        h->slot_bytes = (size_t)align_up(
            std::max<int64_t>({(2 + 2 * (int64_t)h->n) * 8,
                               (int64_t)std::max(h->n_sparse, 1) * (int64_t)sizeof(SparseJob),
                               h->sos.empty() ? 0 : (int64_t)64 << 10}),
            256);
        if (hipHostMalloc(reinterpret_cast<void**>(&h->ring), h->slot_bytes * kRingSlots,
                          hipHostMallocDefault) != hipSuccess) {
            h->ring = nullptr;
            return SHAMPOO_E_HIP;
        }
        for (int i = 0; i < kRingSlots; ++i)
            if (hipEventCreateWithFlags(&h->ring_ev[i], hipEventDisableTiming) != hipSuccess)
                return SHAMPOO_E_HIP;
    }
    for (int i = 0; i < kRingSlots; ++i) h->ring_used[i] = false;
    if (h->roots.size() > 1 && !h->side) {
        // default priority, non-blocking with respect to the null stream
        if (hipStreamCreateWithFlags(&h->side, hipStreamNonBlocking) != hipSuccess) {
            h->side = nullptr;
            return SHAMPOO_E_HIP;
        }
        if (hipEventCreateWithFlags(&h->ev_fork, hipEventDisableTiming) != hipSuccess ||
            hipEventCreateWithFlags(&h->ev_join, hipEventDisableTiming) != hipSuccess)
            return SHAMPOO_E_HIP;
    }
    if ((h->gram.ntiles > 0 || h->gsplit.ntiles > 0) && !h->ovl) {
        if (hipStreamCreateWithFlags(&h->ovl, hipStreamNonBlocking) != hipSuccess) {
            h->ovl = nullptr;
            return SHAMPOO_E_HIP;
        }
        if (hipEventCreateWithFlags(&h->ov_fork, hipEventDisableTiming) != hipSuccess ||
            hipEventCreateWithFlags(&h->ov_join, hipEventDisableTiming) != hipSuccess)
            return SHAMPOO_E_HIP;
    }
    h->async_part = -1;
    // set-up of the allocation-free root pass: this device's static scratch
    if (hipGetDevice(&h->device) != hipSuccess) return SHAMPOO_E_HIP;
    if (noalloc_scratch_ptr(&h->na_ptr) != hipSuccess) return SHAMPOO_E_HIP;
    int rc = hip_err(hipMemsetAsync(h->arena, 0, h->off_tables, s));
    if (rc) return rc;
    rc = hip_err(hipMemcpyAsync(h->arena + h->off_tables, h->blob.bytes.data(), h->blob.bytes.size(),
                                hipMemcpyHostToDevice, s));
    if (rc) return rc;
    if (!h->diag_init.empty()) {
        rc = hip_err(hipMemcpyAsync(h->arena + h->off_diag, h->diag_init.data(),
                                    h->diag_init.size() * sizeof(FactorDiag), hipMemcpyHostToDevice,
                                    s));
        if (rc) return rc;
    }
    rc = hip_err(launch_set_identity(tab<FactorJob>(h, h->ident_jobs_off), (int)h->factors.size(),
                                     at<float>(h, 0), s));
    if (rc) return rc;
    rc = refresh_bases(h, nullptr, nullptr, nullptr, s);  // base 0 (the state buffer) for every kernel
    if (rc) return rc;
    rc = hip_err(hipStreamSynchronize(s));
    if (rc) return rc;
    h->bound = true;
    return SHAMPOO_OK;
}

}  // extern "C"

namespace {
// EMA weights of the statistics: S <- beta2 S + w G G^T, w = 1 - beta2
// (formed in fp64), or a plain sum when beta2 == 1.
GemmArgs stats_args(const shampoo_s* h) {
    const double b2 = h->cfg.beta2;
    GemmArgs a{};
    a.epi = EPI_AXPBY;
    a.alpha = b2 < 1.0 ? 1.0 - b2 : 1.0;
    a.beta = b2;
    return a;
}

int enqueue_sos_stats(shampoo_s* h, const shampoo_sparse_rows* sparse, hipStream_t s);

// Statistics kernels on stream s (pointer table already current).  With
// skip_small the blocks of at most 128 x 128 are left to the fused step
// kernel (enqueue_apply with fused_small).
// The statistics of the two-sided blocks above 128 (the batched GEMM, and the
// column-split partials of a few large blocks with their sum).
int enqueue_stats_big(shampoo_s* h, hipStream_t s) {
    const GemmArgs a = stats_args(h);
    ProfScope ps(h, PC_STATS, s, h->gram.ntiles > 0 || h->gsplit.ntiles > 0);
    int rc = hip_err(launch_gemm_f64_from_f32(tab<GemmTask>(h, h->gram.tasks_off),
                                              tab<TileRef>(h, h->gram.tiles_off), h->gram.ntiles,
                                              at<uint64_t>(h, h->off_bases), a, s));
    if (rc || h->gsplit.ntiles == 0) return rc;
    // a few large blocks: partial products over k, then their fixed-order
    // sum into S = beta2 S + w sum_c part_c
    GemmArgs pa{};
    pa.epi = EPI_STORE;
    pa.alpha = 1.0;
    rc = hip_err(launch_gemm_f64_from_f32(tab<GemmTask>(h, h->gsplit.tasks_off),
                                          tab<TileRef>(h, h->gsplit.tiles_off), h->gsplit.ntiles,
                                          at<uint64_t>(h, h->off_bases), pa, s));
    if (!rc)
        rc = hip_err(launch_sym_reduce(tab<SymReduceJob>(h, h->gred_jobs_off),
                                       tab<TileRef>(h, h->gred_tiles_off), h->n_gred_tiles,
                                       at<double>(h, 0), a.alpha, a.beta, s));
    return rc;
}

// skip_big: the caller runs enqueue_stats_big itself (on another stream).
int enqueue_stats(shampoo_s* h, hipStream_t s, bool skip_small, const shampoo_sparse_rows* sparse,
                  bool skip_big) {
    const GemmArgs a = stats_args(h);
    // fp32 gradients, fp64 products and statistics (exact products; the
    // statistics keep the near-null spectrum that fp32 storage would round
    // into the eps damping)
    if (!skip_small) {
        ProfScope ps(h, PC_STATS_SMALL, s, h->n_gram128 > 0);
        const int rc2 = hip_err(launch_gram128(tab<GramJob>(h, h->gram128_off), h->n_gram128,
                                               at<uint64_t>(h, h->off_bases), at<double>(h, 0),
                                               a.alpha, a.beta, s));
        if (rc2) return rc2;
    }
    if (!skip_big) {
        const int rc2 = enqueue_stats_big(h, s);
        if (rc2) return rc2;
    }
    if (!h->sos.empty()) {
        const int rc = enqueue_sos_stats(h, sparse, s);
        if (rc) return rc;
    }
    if (h->n_symred_tiles == 0) return SHAMPOO_OK;
    // one-sided statistics (Lemma 1): split-K partial products, then their
    // fixed-order sum into S = beta2 S + w sum_c part_c
    ProfScope ps(h, PC_STATS_SPLITK, s);
    GemmArgs pa{};
    pa.epi = EPI_STORE;
    pa.alpha = 1.0;
    pa.beta = 0.0;
    int rc = hip_err(launch_gemm_f64_from_f32(tab<GemmTask>(h, h->splitk.tasks_off),
                                              tab<TileRef>(h, h->splitk.tiles_off), h->splitk.ntiles,
                                              at<uint64_t>(h, h->off_bases), pa, s));
    if (rc) return rc;
    return hip_err(launch_sym_reduce(tab<SymReduceJob>(h, h->symred_jobs_off),
                                     tab<TileRef>(h, h->symred_tiles_off), h->n_symred_tiles,
                                     at<double>(h, 0), a.alpha, a.beta, s));
}

int check_stats_args(const shampoo_s* h, const float* const* grads,
                     const shampoo_sparse_rows* sparse) {
    if (!grads) return SHAMPOO_E_ARG;
    for (auto& bp : h->blocks)
        if (h->tensors[bp.tensor].mode != 2 && !grads[bp.tensor]) return SHAMPOO_E_ARG;
    if (!h->sos.empty() && !sparse) return SHAMPOO_E_ARG;
    for (const SosPlan& sp : h->sos) {
        const shampoo_sparse_rows& sr = sparse[sp.tensor];
        if (sr.n_rows < 0 || sr.n_rows > h->tensors[sp.tensor].rows) return SHAMPOO_E_ARG;
        if (sr.n_rows > 0 && (!sr.rows || !sr.row_grads)) return SHAMPOO_E_ARG;
    }
    return SHAMPOO_OK;
}

int check_apply_args(const shampoo_s* h, float* const* params, const float* const* grads,
                     const shampoo_sparse_rows* sparse) {
    if (!params || !grads) return SHAMPOO_E_ARG;
    for (int t = 0; t < h->n; ++t) {
        if (!params[t]) return SHAMPOO_E_ARG;
        if (h->tensors[t].mode != 2 && !grads[t]) return SHAMPOO_E_ARG;
    }
    if (h->n_sparse > 0 && !sparse) return SHAMPOO_E_ARG;
    for (const SosPlan& sp : h->sos) {
        const shampoo_sparse_rows& sr = sparse[sp.tensor];
        if (sr.n_rows < 0 || sr.n_rows > h->tensors[sp.tensor].rows) return SHAMPOO_E_ARG;
        if (sr.n_rows > 0 && (!sr.rows || !sr.row_grads)) return SHAMPOO_E_ARG;
    }
    return SHAMPOO_OK;
}

int enqueue_apply(shampoo_s* h, float* const* params, const shampoo_sparse_rows* sparse,
                  hipStream_t s, bool fused_small);
int enqueue_sos_apply(shampoo_s* h, float* const* params, const shampoo_sparse_rows* sparse,
                      hipStream_t s);
}  // namespace

extern "C" {

int shampoo_update_stats(shampoo_t* h, const float* const* grads,
                         const shampoo_sparse_rows* sparse, void* stream) {
    if (!h || !grads) return SHAMPOO_E_ARG;
    if (!h->bound) return SHAMPOO_E_STATE;
    int rc = check_stats_args(h, grads, sparse);
    if (rc) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    rc = refresh_bases(h, grads, nullptr, sparse, s);
    if (rc) return rc;
    return enqueue_stats(h, s, false, sparse, false);
}

namespace {
// scr: the chain's iterate scratch, or null for the state buffer's own.
int run_newton(shampoo_s* h, std::vector<NewtonChunk>& chunks, bool fp64, const int32_t* gate,
               int gate_val, int32_t* prec, hipStream_t s, unsigned char* scr = nullptr) {
    NewtonArgs na{};
    na.is_fp64 = fp64 ? 1 : 0;
    na.gate = gate;
    na.gate_val = gate_val;
    na.chk = at<unsigned long long>(h, h->off_chk);
    void* scratch = scr ? scr : h->arena + (fp64 ? h->off_scr64 : h->off_scr32);
    FactorDiag* diag = at<FactorDiag>(h, h->off_diag);
    GemmArgs g{};
    g.epi = EPI_STORE;
    g.alpha = 1.0;
    g.beta = 0.0;
    g.gate = gate;
    g.gate_val = gate_val;
    const uint64_t* bases = at<uint64_t>(h, h->off_bases);
    for (auto& ch : chunks) {
        const int p = ch.p;
        na.p = p;
        // with a convergence exit (newton_tol > 0) the chain takes the scaled
        // steps and stops after the one where every eigenvalue of M is within
        // newton_tol of 1 by the schedule's bound: one step after in fp32
        // (the error is then about (p+1)/(2p) tol^2, 6e-7 for 1e-3, and the
        // root's about that over p, at fp32 rounding), two in fp64 (about
        // 0.24 tol^4); without an eps floor there is no bound: the full count
        const bool scaled = h->cfg.newton_tol > 0.0 && h->cfg.eps_rel > 0.0 && !ch.fused;
        std::vector<double> mu(ch.iters, 1.0);
        int conv_steps = ch.iters;
        if (scaled)
            newton_schedule(p, h->cfg.eps_rel, ch.iters, h->cfg.newton_tol, fp64 ? 2 : 1, mu,
                            conv_steps);
        const int iters = std::min(ch.iters, conv_steps);
        na.iters = iters;
        auto set_step = [&](int it) {
            g.xc1 = std::pow(mu[it], 1.0 / p) * (p + 1) / p;
            g.xc2 = -std::pow(mu[it], 1.0 + 1.0 / p) / p;
        };
        set_step(0);
        na.xc1 = g.xc1;
        na.xc2 = g.xc2;
        // a packed chain reads the slot jobs written by k_route_compact and
        // gates its products by the slot flags
        const FactorJob* jobs = ch.compact ? at<FactorJob>(h, ch.slot_jobs_off)
                                           : tab<FactorJob>(h, ch.jobs_off);
        na.gate = ch.compact ? nullptr : gate;
        g.gate = ch.compact ? at<int32_t>(h, h->off_slot_live) : gate;
        g.gate_val = ch.compact ? 1 : gate_val;
        int rc;
        if (ch.fused) {
            // lambda_max, eps, the root and the kappa estimate of every factor
            // up to 128 in one kernel
            FusedArgs fa{};
            fa.p = p;
            fa.iters = ch.iters;
            // lambda_max: lanczos_steps steps, or (0) until the top Ritz
            // residual is within kLanczosTol, at most 64 steps
            fa.steps_s = h->cfg.lanczos_steps > 0 ? h->cfg.lanczos_steps : 64;
            fa.lz_tol = h->cfg.lanczos_steps > 0 ? 0.0 : kLanczosTol;
            fa.steps_p = h->cfg.lanczos_steps > 0 ? std::min(h->cfg.lanczos_steps, 8) : 8;
            fa.auto_route = h->cfg.root_mode == SHAMPOO_ROOT_AUTO ? 1 : 0;
            fa.eps_rel = h->cfg.eps_rel;
            fa.threshold = h->cfg.fp64_cond_threshold;
            fa.tol = (float)h->cfg.newton_tol;
            ProfScope ps(h, PC_NEWTON_FUSED, s);
            rc = hip_err(launch_newton128(jobs, ch.njobs, at<double>(h, 0), at<float>(h, 0), diag,
                                          prec, fa, s));
            if (rc) return rc;
            continue;
        }
        {
            ProfScope ps(h, PC_NEWTON_INIT, s);
            rc = hip_err(launch_newton_init(fp64, jobs, ch.njobs, ch.ld, at<double>(h, 0), scratch, diag,
                                            na, s));
        }
        if (rc) return rc;
        {
            // timing scopes per launch: products, split-K sums and
            // convergence checks are separate kernel families
            static const std::vector<NewtonStage> kNone;
            for (int it = 0; it < iters; ++it) {
                set_step(it);
                // the last step forms X only (M_iters is never read); a single
                // step is the start's X_1 alone
                const bool last = it == iters - 1;
                const std::vector<NewtonStage>& stg =
                    it == 0 ? (last ? kNone : ch.first) : (last ? ch.last[it & 1] : ch.stages[it & 1]);
                for (const NewtonStage& S : stg) {
                    const GemmTask* tk = tab<GemmTask>(h, S.gemm.tasks_off);
                    const TileRef* tl = tab<TileRef>(h, S.gemm.tiles_off);
                    g.persist = (fp64 && S.sorted) ? kPersistGrid : 0;
                    g.chain = S.chain;
                    {
                        ProfScope ps(h, fp64 ? PC_NEWTON_GEMM64 : PC_NEWTON_GEMM32, s);
                        rc = hip_err(fp64 ? launch_gemm_f64(tk, tl, S.gemm.ntiles, bases, g, s)
                                          : launch_gemm_f32(tk, tl, S.gemm.ntiles, bases, g, s));
                    }
                    if (!rc && S.parts > 1) {
                        ProfScope ps(h, PC_NEWTON_SPLIT, s);
                        rc = hip_err(launch_split_sum(fp64, tab<SplitSumJob>(h, S.sum_jobs_off),
                                                      tab<TileRef>(h, S.sum_tiles_off), S.sum_ntiles,
                                                      h->arena, g.gate, g.gate_val, s));
                    }
                    if (rc) return rc;
                }
            }
        }
        // the final X sits in buffer (iters % 2) of each slot, the last M
        // formed (M_{iters-1}, from which the last T came) in the other
        ProfScope ps(h, PC_NEWTON_COMMIT, s);
        const size_t mat_bytes = (size_t)ch.ld * ch.ld * (fp64 ? 8 : 4);
        rc = hip_err(launch_newton_commit(fp64, jobs, ch.njobs, ch.ld, at<float>(h, 0),
                                          static_cast<unsigned char*>(scratch) + (size_t)(iters & 1) * mat_bytes,
                                          static_cast<unsigned char*>(scratch) +
                                              (size_t)((iters - 1) & 1) * mat_bytes,
                                          diag, na, s));
        if (rc) return rc;
    }
    return SHAMPOO_OK;
}
}  // namespace

}  // extern "C"

namespace {
// One root pass over the factors of rt (every factor, or one part of a
// staggered pass).
int enqueue_roots(shampoo_s* h, RootTables& rt, hipStream_t s, unsigned char* scr = nullptr) {
    const int nf = (int)h->factors.size();
    if (nf == 0) return SHAMPOO_OK;
    const shampoo_config& c = h->cfg;
    FactorDiag* diag = at<FactorDiag>(h, h->off_diag);
    int32_t* prec = at<int32_t>(h, h->off_prec);
    LanczosArgs la{};
    la.steps = c.lanczos_steps > 0 ? c.lanczos_steps : 64;
    la.tol = c.lanczos_steps > 0 ? 0.0 : kLanczosTol;
    la.mode = 0;
    la.eps_rel = c.eps_rel;
    la.threshold = c.fp64_cond_threshold;
    la.diag = diag;
    la.prec = prec;
    la.work = at<double>(h, h->off_lzwork);
    la.route_all_fp64 = c.root_mode == SHAMPOO_ROOT_F64 ? 1 : 0;
    LanczosArgs lp = la;
    lp.mode = 1;
    lp.steps = std::min(la.steps, 8);  // kappa estimate: a factor-2 decision
    lp.tol = 0.0;
    int rc = SHAMPOO_OK;
    auto lanczos = [&](int64_t small_off, int64_t big_off, bool on_stats, bool with_small,
                       const LanczosArgs& a) -> int {
        const void* base = h->arena;
        ProfScope ps(h, on_stats ? PC_LANCZOS_S : PC_LANCZOS_P, s,
                     rt.n_lanczos_big > 0 || (with_small && rt.n_lanczos_small > 0));
        int r = SHAMPOO_OK;
        if (with_small)
            r = hip_err(launch_lanczos(tab<LanczosJob>(h, small_off), rt.n_lanczos_small, base,
                                       on_stats, false, a, s));
        if (r) return r;
        LanczosArgs ab = a;
        ab.max_n = rt.lanczos_big_max_n;
        return hip_err(launch_lanczos(tab<LanczosJob>(h, big_off), rt.n_lanczos_big, base, on_stats,
                                      true, ab, s));
    };
    if (use_fp32(c)) {
        // factors up to 128: everything inside the fused kernel; larger ones:
        // Lanczos on S, batched fp32 Newton, Lanczos on the root
        rc = lanczos(rt.lanczos_s_small_off, rt.lanczos_s_big_off, true, false, la);
        if (rc) return rc;
        rc = run_newton(h, rt.chunks32, false, nullptr, 0, prec, s, scr);
        if (rc) return rc;
        lp.auto_route = c.root_mode == SHAMPOO_ROOT_AUTO ? 1 : 0;
        rc = lanczos(rt.lanczos_p_small_off, rt.lanczos_p_big_off, false, false, lp);
        if (rc) return rc;
        if (c.root_mode == SHAMPOO_ROOT_AUTO) {
            {
                ProfScope ps(h, PC_ROUTE, s, !rt.compact.empty());
                rc = hip_err(launch_route_compact(tab<CompactClass>(h, rt.compact_off),
                                                  (int)rt.compact.size(),
                                                  tab<FactorJob>(h, h->slot_tmpl_off), prec, 1,
                                                  at<FactorJob>(h, h->off_slot_jobs),
                                                  at<int32_t>(h, h->off_slot_live), s));
            }
            if (rc) return rc;
            rc = run_newton(h, rt.chunks64, true, prec, 1, prec, s, scr);
        }
        return rc;
    }
    // all fp64
    LanczosArgs la_small = la;
    la_small.steps = c.lanczos_steps > 0 ? c.lanczos_steps : 64;
    {
        ProfScope ps(h, PC_LANCZOS_S, s);
        rc = hip_err(launch_lanczos(tab<LanczosJob>(h, rt.lanczos_s_small_off), rt.n_lanczos_small,
                                    h->arena, true, false, la_small, s));
        LanczosArgs lb = la;
        lb.max_n = rt.lanczos_big_max_n;
        if (!rc)
            rc = hip_err(launch_lanczos(tab<LanczosJob>(h, rt.lanczos_s_big_off), rt.n_lanczos_big,
                                        h->arena, true, true, lb, s));
    }
    if (rc) return rc;
    rc = run_newton(h, rt.chunks64, true, nullptr, 1, prec, s, scr);
    if (rc) return rc;
    lp.auto_route = 0;
    return lanczos(rt.lanczos_p_small_off, rt.lanczos_p_big_off, false, true, lp);
}
}  // namespace

extern "C" {

int shampoo_compute_inverse_roots(shampoo_t* h, void* stream) {
    if (!h) return SHAMPOO_E_ARG;
    if (!h->bound || h->async_part >= 0) return SHAMPOO_E_STATE;
    return enqueue_roots(h, h->roots[0], static_cast<hipStream_t>(stream));
}

int shampoo_compute_inverse_roots_noalloc(shampoo_t* h, void* stream) {
    if (!h) return SHAMPOO_E_ARG;
    if (!h->bound || h->async_part >= 0 || !h->na_ptr) return SHAMPOO_E_STATE;
    if (!h->noalloc_ok) return SHAMPOO_E_UNSUPPORTED;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return SHAMPOO_E_HIP;
    if (dev != h->device) return SHAMPOO_E_STATE;
    // no timing events here (creating one may allocate)
    const bool prof = h->prof_on;
    h->prof_on = false;
    const int rc = enqueue_roots(h, h->roots_na, static_cast<hipStream_t>(stream),
                                 static_cast<unsigned char*>(h->na_ptr));
    h->prof_on = prof;
    return rc;
}

int shampoo_compute_inverse_roots_part(shampoo_t* h, int32_t part, void* stream) {
    if (!h) return SHAMPOO_E_ARG;
    const int nparts = (int)h->roots.size() - 1;
    if (nparts < 1 || part < 0 || part >= nparts) return SHAMPOO_E_ARG;
    if (!h->bound || h->async_part >= 0) return SHAMPOO_E_STATE;
    return enqueue_roots(h, h->roots[1 + part], static_cast<hipStream_t>(stream));
}

int shampoo_roots_async_begin(shampoo_t* h, int32_t part, void* stream) {
    if (!h) return SHAMPOO_E_ARG;
    const int nparts = (int)h->roots.size() - 1;
    if (nparts < 1 || part < 0 || part >= nparts) return SHAMPOO_E_ARG;
    if (!h->bound || h->async_part >= 0) return SHAMPOO_E_STATE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    // snapshot of the part's statistics and current roots, in stream order
    int rc = hip_err(launch_copy_jobs(tab<CopyJob>(h, h->async_begin_off[part]), h->async_begin_n[part],
                                      h->arena, s));
    if (!rc) rc = hip_err(hipEventRecord(h->ev_fork, s));
    if (!rc) rc = hip_err(hipStreamWaitEvent(h->side, h->ev_fork, 0));
    if (rc) return rc;
    // the root pass of the part on the library's stream: it reads the
    // snapshot and writes the staged roots (and the part's diagnostics)
    rc = enqueue_roots(h, h->async_roots[part], h->side);
    const int rc_ev = hip_err(hipEventRecord(h->ev_join, h->side));
    if (rc) return rc;
    if (rc_ev) return rc_ev;
    h->async_part = part;
    return SHAMPOO_OK;
}

int shampoo_roots_async_end(shampoo_t* h, void* stream) {
    if (!h) return SHAMPOO_E_ARG;
    if (!h->bound) return SHAMPOO_E_STATE;
    if (h->async_part < 0) return SHAMPOO_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int q = h->async_part;
    int rc = hip_err(hipStreamWaitEvent(s, h->ev_join, 0));
    if (!rc) rc = hip_err(launch_copy_jobs(tab<CopyJob>(h, h->async_end_off[q]), h->async_end_n[q],
                                           h->arena, s));
    if (rc) return rc;
    h->async_part = -1;
    return SHAMPOO_OK;
}

int shampoo_precondition_and_apply(shampoo_t* h, float* const* params, const float* const* grads,
                                   const shampoo_sparse_rows* sparse, void* stream) {
    if (!h || !params || !grads) return SHAMPOO_E_ARG;
    if (!h->bound) return SHAMPOO_E_STATE;
    int rc = check_apply_args(h, params, grads, sparse);
    if (rc) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    rc = refresh_bases(h, grads, params, sparse, s);
    if (rc) return rc;
    return enqueue_apply(h, params, sparse, s, false);
}

int shampoo_step(shampoo_t* h, float* const* params, const float* const* grads,
                 const shampoo_sparse_rows* sparse, int32_t roots, void* stream) {
    if (!h || !params || !grads) return SHAMPOO_E_ARG;
    const int nparts = (int)h->roots.size() - 1;
    if (roots != SHAMPOO_ROOTS_NONE && roots != SHAMPOO_ROOTS_ALL && (roots < 0 || roots >= nparts))
        return SHAMPOO_E_ARG;
    if (!h->bound || (roots != SHAMPOO_ROOTS_NONE && h->async_part >= 0)) return SHAMPOO_E_STATE;
    int rc = check_stats_args(h, grads, sparse);
    if (!rc) rc = check_apply_args(h, params, grads, sparse);
    if (rc) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    rc = refresh_bases(h, grads, params, sparse, s);
    if (rc) return rc;
    if (roots != SHAMPOO_ROOTS_NONE) {
        // the roots need this step's statistics, the apply needs the roots
        rc = enqueue_stats(h, s, false, sparse, false);
        if (!rc) rc = enqueue_roots(h, h->roots[roots == SHAMPOO_ROOTS_ALL ? 0 : 1 + roots], s);
        if (!rc) rc = enqueue_apply(h, params, sparse, s, false);
        return rc;
    }
    // no root pass: statistics and apply of each block <= 128 share one
    // kernel, and the statistics of the larger blocks (fp64 MFMA) run on a
    // second stream beside the apply (bf16 products and streaming), with
    // which they share only read-only inputs; the step ends when both have
    // (with per-launch profiling on, in order on one stream: each launch is
    // then timed alone)
    const bool ovl = h->ovl && !h->prof_on && (h->gram.ntiles > 0 || h->gsplit.ntiles > 0);
    if (ovl) {
        rc = hip_err(hipEventRecord(h->ov_fork, s));
        if (!rc) rc = hip_err(hipStreamWaitEvent(h->ovl, h->ov_fork, 0));
        if (rc) return rc;   // nothing on the second stream
        rc = enqueue_stats_big(h, h->ovl);
        const int rj = hip_err(hipEventRecord(h->ov_join, h->ovl));
        if (rj) return rj;
        if (rc) {
            (void)hipStreamWaitEvent(s, h->ov_join, 0);
            return rc;
        }
    }
    rc = enqueue_stats(h, s, true, sparse, ovl);
    if (!rc) rc = enqueue_apply(h, params, sparse, s, true);
    if (ovl) {
        const int rj = hip_err(hipStreamWaitEvent(s, h->ov_join, 0));
        if (!rc) rc = rj;
    }
    return rc;
}

}  // extern "C"

namespace {
// Sparse-row tables with one-sided preconditioning (Lemma 1, R side): the
// statistics of this call's listed rows, S <- beta2 S + w g^T g.  The rows
// are cut into at most kSosMaxChunks chunks of at least kSosMinRows rows;
// each chunk's product goes to its own fp64 partial and k_sym_reduce sums
// them in chunk order (with no rows, S only decays).  Per-call tables go
// through the staging ring into the state buffer.
int enqueue_sos_stats(shampoo_s* h, const shampoo_sparse_rows* sparse, hipStream_t s) {
    std::vector<GemmTask> tasks;
    std::vector<SymReduceJob> red;
    std::vector<TileRef> rtiles;
    for (const SosPlan& sp : h->sos) {
        const FactorPlan& f = h->factors[sp.factor];
        const TensorPlan& tp = h->tensors[sp.tensor];
        const int64_t n = sparse[sp.tensor].n_rows;
        int chunks = 0;
        if (n > 0) {
            const int want = std::min<int>(kSosMaxChunks, ceil_div(n, kSosMinRows));
            const int64_t len = align_up(ceil_div(n, want), 32);
            chunks = ceil_div(n, len);
            for (int ck = 0; ck < chunks; ++ck) {
                GemmTask t{};
                const int64_t k0 = (int64_t)ck * len;
                t.a_base = t.b_base = 1 + sp.tensor;   // the row gradients (n x cols)
                t.a_off = t.b_off = k0 * tp.cols;
                t.lda = t.ldb = (int)tp.cols;
                t.c_base = 0;
                t.c_off = sp.part_off / 8 + (int64_t)ck * f.ld * f.ld;
                t.ldc = f.ld;
                t.M = t.N = f.dim;
                t.K = (int)std::min<int64_t>(len, n - k0);
                t.tiles_n = ceil_div(t.N, kTile);
                t.trans = 1 | 16 | band_bit(t.tiles_n);
                t.factor = -1;
                t.norm_slot = -1;
                tasks.push_back(t);
            }
        }
        SymReduceJob r{};
        r.part_off = sp.part_off / 8;
        r.s_off = f.off_s / 8;
        r.nparts = chunks;
        r.dim = f.dim;
        r.ld = f.ld;
        r.tiles = ceil_div(f.dim, 32);
        for (int a = 0; a < r.tiles; ++a)
            for (int b = a; b < r.tiles; ++b) rtiles.push_back({(int32_t)red.size(), a * r.tiles + b});
        red.push_back(r);
    }
    Blob b;
    const LaunchRef L = add_launch(b, tasks);
    const int64_t o_red = b.add(red), o_rtiles = b.add(rtiles);
    int rc = stage_upload(h, b.bytes.data(), b.bytes.size(), h->off_sos_stats, s);
    if (rc) return rc;
    const GemmArgs a = stats_args(h);
    GemmArgs pa{};
    pa.epi = EPI_STORE;
    pa.alpha = 1.0;
    pa.beta = 0.0;
    ProfScope ps(h, PC_SOS_STATS, s);
    rc = hip_err(launch_gemm_f64_from_f32(at<GemmTask>(h, h->off_sos_stats + L.tasks_off),
                                          at<TileRef>(h, h->off_sos_stats + L.tiles_off), L.ntiles,
                                          at<uint64_t>(h, h->off_bases), pa, s));
    if (rc) return rc;
    return hip_err(launch_sym_reduce(at<SymReduceJob>(h, h->off_sos_stats + o_red),
                                     at<TileRef>(h, h->off_sos_stats + o_rtiles), (int)rtiles.size(),
                                     at<double>(h, 0), a.alpha, a.beta, s));
}

// The apply of the sparse one-sided tables for this call: a += g*g and
// ||A||^2 over the listed rows, D = g P_R with ||D||^2 per tile, the graft
// scale over the table, then W_r -= lr s D_r on the listed rows.
int enqueue_sos_apply(shampoo_s* h, float* const* params, const shampoo_sparse_rows* sparse,
                      hipStream_t s) {
    const shampoo_config& c = h->cfg;
    std::vector<SosJob> jobs;
    std::vector<GemmTask> tasks;
    std::vector<BlockNorms> bns;
    int chunks = 0;
    for (const SosPlan& sp : h->sos) {
        const TensorPlan& tp = h->tensors[sp.tensor];
        const FactorPlan& f = h->factors[sp.factor];
        const BlockPlan& bp = h->blocks[sp.block];
        const shampoo_sparse_rows& sr = sparse[sp.tensor];
        const int64_t n = sr.n_rows;
        const int rows_per = (int)std::max<int64_t>(1, kElemChunk / tp.cols);
        const int nch = n > 0 ? ceil_div(n, rows_per) : 0;
        SosJob j{};
        j.rows_ptr = reinterpret_cast<int64_t>(sr.rows);
        j.grads_ptr = reinterpret_cast<int64_t>(sr.row_grads);
        j.w_ptr = reinterpret_cast<int64_t>(params[sp.tensor]);
        j.a_off = tp.off_a / 4;
        j.d_off = tp.off_d / 4;
        j.n_rows = n;
        j.table_rows = tp.rows;
        j.cols = (int)tp.cols;
        j.chunk_rows = rows_per;
        j.first_chunk = chunks;
        j.slot_a = bp.a_slot;
        j.block = sp.block;
        j.vec = (tp.cols % 4 == 0) && ((reinterpret_cast<uintptr_t>(sr.row_grads) & 15) == 0) &&
                ((reinterpret_cast<uintptr_t>(params[sp.tensor]) & 15) == 0);
        jobs.push_back(j);
        chunks += nch;
        int d_tiles = 0;
        if (n > 0) {
            GemmTask u{};
            u.a_base = 1 + sp.tensor; u.a_off = 0; u.lda = (int)tp.cols;   // g (n x cols)
            u.b_base = 0; u.b_off = f.off_p / 4; u.ldb = f.ld;
            u.c_base = 0; u.c_off = tp.off_d / 4; u.ldc = (int)tp.cols;
            u.M = (int)n; u.N = (int)tp.cols; u.K = (int)tp.cols;
            u.trans = 0;
            u.tiles_n = ceil_div(u.N, kTile);
            u.factor = -1;
            u.norm_slot = bp.d_slot;
            tasks.push_back(u);
            d_tiles = ceil_div(n, kTile) * u.tiles_n;
        }
        bns.push_back({bp.a_slot, nch, bp.d_slot, d_tiles, sp.block, 0});
    }
    Blob b;
    const int64_t o_jobs = b.add(jobs);
    const LaunchRef L = add_launch(b, tasks);
    const int64_t o_bn = b.add(bns);
    int rc = stage_upload(h, b.bytes.data(), b.bytes.size(), h->off_sos_apply, s);
    if (rc) return rc;
    const SosJob* dj = at<SosJob>(h, h->off_sos_apply + o_jobs);
    float* arena = at<float>(h, 0);
    double* partA = at<double>(h, h->off_partA);
    double* partD = at<double>(h, h->off_partD);
    float* scale = at<float>(h, h->off_scale);
    {
        ProfScope ps(h, PC_SOS_NORM, s, chunks > 0);
        rc = hip_err(launch_sos_norm(dj, (int)jobs.size(), chunks, arena, (float)c.graft_eps, partA, s));
    }
    if (rc) return rc;
    GemmArgs g{};
    g.epi = EPI_STORE;
    g.alpha = 1.0;
    g.norms = partD;
    {
        ProfScope ps(h, PC_SOS_APPLY, s, L.ntiles > 0);
        rc = hip_err(launch_gemm_f32(at<GemmTask>(h, h->off_sos_apply + L.tasks_off),
                                     at<TileRef>(h, h->off_sos_apply + L.tiles_off), L.ntiles,
                                     at<uint64_t>(h, h->off_bases), g, s, 2));
    }
    if (rc) return rc;
    {
        ProfScope ps(h, PC_SCALE, s);
        rc = hip_err(launch_block_scale(at<BlockNorms>(h, h->off_sos_apply + o_bn), (int)bns.size(),
                                        partA, partD, scale, s));
    }
    if (rc) return rc;
    ProfScope ps(h, PC_SOS_UPDATE, s, chunks > 0);
    return hip_err(launch_sos_update(dj, (int)jobs.size(), chunks, arena, scale, (float)c.lr, s));
}

// Apply kernels on stream s (pointer table already current).  fused_small:
// the blocks of at most 128 x 128 go through the fused step kernel, which
// also updates their statistics.
int enqueue_apply(shampoo_s* h, float* const* params, const shampoo_sparse_rows* sparse,
                  hipStream_t s, bool fused_small) {
    int rc = SHAMPOO_OK;
    const uint64_t* bases = at<uint64_t>(h, h->off_bases);
    float* arena = at<float>(h, 0);
    double* partA = at<double>(h, h->off_partA);
    double* partD = at<double>(h, h->off_partD);
    float* scale = at<float>(h, h->off_scale);
    const shampoo_config& c = h->cfg;
    const UpdateArgs ua{(float)c.beta1, (float)c.lr, (float)c.graft_eps};

    {
        ProfScope ps(h, PC_ADAGRAD, s, h->n_blockchunks > 0);
        rc = hip_err(launch_adagrad_norm(tab<BlockChunk>(h, h->blockchunks_off), h->n_blockchunks, bases,
                                     arena, (float)c.graft_eps, partA, s));
    }
    if (rc) return rc;
    // the fused step's launch also takes the dense-Adagrad rows
    const bool fold = fused_small && h->n_apply128 > 0 && h->n_fold > 0;
    if (fused_small) {
        const GemmArgs sa = stats_args(h);
        ProfScope ps(h, PC_STEP_FUSED, s, h->n_apply128 > 0);
        rc = hip_err(launch_step128(tab<StepJob>(h, h->step128_off), h->n_apply128,
                                    tab<RowChunk>(h, h->fold_off), fold ? h->n_fold : 0, h->n, bases,
                                    arena, sa.alpha, sa.beta, (float)c.graft_eps, partA, partD, ua, s));
    } else {
        ProfScope ps(h, PC_APPLY_FUSED, s, h->n_apply128 > 0);
        rc = hip_err(launch_apply128(tab<ApplyJob>(h, h->apply128_off), h->n_apply128, bases, arena,
                                     (float)c.graft_eps, partA, partD, ua, s));
    }
    if (rc) return rc;
    if (h->nt1.ntiles > 0 || h->nt2.ntiles > 0) {
        // split precision: T^T = P_R G^T (with the Adagrad pass), D = P_L T
        NtArgs na{partD, partA, arena, (float)c.graft_eps};
        {
            ProfScope ps(h, PC_APPLY_T, s, h->nt1.ntiles > 0);
            rc = hip_err(launch_gemm_nt3(tab<NtTask>(h, h->nt1.tasks_off),
                                         tab<TileRef>(h, h->nt1.tiles_off), h->nt1.ntiles, bases,
                                         na, true, s));
        }
        if (rc) return rc;
        {
            ProfScope ps(h, PC_APPLY_D, s, h->nt2.ntiles > 0);
            rc = hip_err(launch_gemm_nt3(tab<NtTask>(h, h->nt2.tasks_off),
                                         tab<TileRef>(h, h->nt2.tiles_off), h->nt2.ntiles, bases,
                                         na, false, s));
        }
        if (rc) return rc;
    }
    GemmArgs g{};
    g.epi = EPI_STORE;
    g.alpha = 1.0;
    g.norms = partD;
    {
        ProfScope ps(h, PC_APPLY_T, s, h->apply1.ntiles > 0);
        rc = hip_err(launch_gemm_f32(tab<GemmTask>(h, h->apply1.tasks_off),
                                     tab<TileRef>(h, h->apply1.tiles_off), h->apply1.ntiles, bases, g, s,
                                     1));
    }
    if (rc) return rc;
    {
        ProfScope ps(h, PC_APPLY_D, s, h->apply2.ntiles > 0);
        rc = hip_err(launch_gemm_f32(tab<GemmTask>(h, h->apply2.tasks_off),
                                     tab<TileRef>(h, h->apply2.tiles_off), h->apply2.ntiles, bases, g, s,
                                     2));
    }
    if (rc) return rc;
    {
        ProfScope ps(h, PC_SCALE, s, h->n_blocknorms > 0);
        rc = hip_err(launch_block_scale(tab<BlockNorms>(h, h->blocknorms_off), h->n_blocknorms,
                                        partA, partD, scale, s));
    }
    if (rc) return rc;
    {
        const int n = fold ? h->n_shampoo_rows : h->n_rowchunks;
        ProfScope ps(h, PC_UPDATE, s, n > 0);
        rc = hip_err(launch_update(tab<RowChunk>(h, fold ? h->shampoo_rows_off : h->rowchunks_off), n,
                                   bases, h->n, arena, scale, ua, s));
    }
    if (rc) return rc;
    if (!h->sos.empty()) {
        rc = enqueue_sos_apply(h, params, sparse, s);
        if (rc) return rc;
    }
    if (h->n_sparse > 0) {
        std::vector<SparseJob> jobs;
        int64_t items = 0;
        for (int t = 0; t < h->n; ++t) {
            const TensorPlan& tp = h->tensors[t];
            if (tp.mode != 2 || tp.os_side >= 0) continue;
            const shampoo_sparse_rows& sr = sparse[t];
            if (sr.n_rows < 0 || sr.n_rows > tp.rows) return SHAMPOO_E_ARG;
            if (sr.n_rows == 0) continue;
            if (!sr.rows || !sr.row_grads) return SHAMPOO_E_ARG;
            SparseJob j{};
            j.rows_ptr = reinterpret_cast<int64_t>(sr.rows);
            j.grads_ptr = reinterpret_cast<int64_t>(sr.row_grads);
            j.w_ptr = reinterpret_cast<int64_t>(params[t]);
            j.a_off = tp.off_a / 4;
            j.n_rows = sr.n_rows;
            j.table_rows = tp.rows;
            j.cols = (int)tp.cols;
            j.vec = (tp.cols % 4 == 0) && ((reinterpret_cast<uintptr_t>(sr.row_grads) & 15) == 0) &&
                    ((reinterpret_cast<uintptr_t>(params[t]) & 15) == 0);
            j.first_item = items;
            items += sr.n_rows * (j.vec ? tp.cols / 4 : tp.cols);
            jobs.push_back(j);
        }
        if (!jobs.empty()) {
            rc = stage_upload(h, jobs.data(), jobs.size() * sizeof(SparseJob), h->off_sparse, s);
            if (rc) return rc;
            ProfScope ps(h, PC_SPARSE, s);
            rc = hip_err(launch_sparse_rows(at<SparseJob>(h, h->off_sparse), (int)jobs.size(), items,
                                            arena, (float)c.lr, (float)c.graft_eps, s));
            if (rc) return rc;
        }
    }
    return SHAMPOO_OK;
}
}  // namespace

extern "C" {

int shampoo_get_diagnostics(shampoo_t* h, shampoo_factor_diag* out, int32_t cap, void* stream) {
    if (!h || (!out && cap > 0) || cap < 0) return SHAMPOO_E_ARG;
    if (!h->bound) return SHAMPOO_E_STATE;
    static_assert(sizeof(shampoo_factor_diag) == sizeof(FactorDiag), "diag layout");
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int n = std::min<int>(cap, (int)h->factors.size());
    if (n > 0) {
        int rc = hip_err(hipMemcpyAsync(out, h->arena + h->off_diag, (size_t)n * sizeof(FactorDiag),
                                        hipMemcpyDeviceToHost, s));
        if (rc) return rc;
    }
    return hip_err(hipStreamSynchronize(s));
}

int shampoo_profile_enable(shampoo_t* h, int32_t on) {
    if (!h) return SHAMPOO_E_ARG;
    h->prof_on = on != 0;
    return SHAMPOO_OK;
}

int shampoo_profile_read(shampoo_t* h, shampoo_kernel_time* out, int32_t cap, int32_t* n_out) {
    if (!h || cap < 0 || (!out && cap > 0)) return SHAMPOO_E_ARG;
    int rc = SHAMPOO_OK;
    for (auto& r : h->prof_pending) {
        float ms = 0.f;
        if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess)
            rc = SHAMPOO_E_HIP;
        h->prof_launches[r.cat] += 1;
        h->prof_ms[r.cat] += ms;
        h->prof_pool.push_back(r.a);
        h->prof_pool.push_back(r.b);
    }
    h->prof_pending.clear();
    const int n = std::min<int>(cap, PC_COUNT);
    for (int i = 0; i < n; ++i) {
        std::memset(out[i].name, 0, sizeof(out[i].name));
        std::strncpy(out[i].name, kProfNames[i], sizeof(out[i].name) - 1);
        out[i].launches = h->prof_launches[i];
        out[i].total_ms = h->prof_ms[i];
    }
    if (n_out) *n_out = n;
    for (int i = 0; i < PC_COUNT; ++i) {
        h->prof_launches[i] = 0;
        h->prof_ms[i] = 0.0;
    }
    return rc;
}

void shampoo_destroy(shampoo_t* h) { delete h; }

const char* shampoo_strerror(int status) {
    switch (status) {
        case SHAMPOO_OK: return "ok";
        case SHAMPOO_E_ARG: return "invalid argument";
        case SHAMPOO_E_STATE: return "state not bound or too small";
        case SHAMPOO_E_HIP: return "HIP runtime or launch error";
        case SHAMPOO_E_NOMEM: return "host allocation failed";
        case SHAMPOO_E_UNSUPPORTED: return "unsupported configuration";
        default: return "unknown status";
    }
}

}  // extern "C"
