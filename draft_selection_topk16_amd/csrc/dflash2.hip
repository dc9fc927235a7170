// MI355X (gfx950) DFlash 2 path selector: kernels and the C ABI declared in
// include/dflash2.h.
//
// The selector ("DFlash 2: Keep Drafting Parallel", section "A Lightweight
// Path Selector") keeps the top-K candidates per draft position, scores every
// adjacent pair with S_t(a,b) = U_t(b) + <A(a) (.) H(h_t), B(b)>, and walks
// the scores once from the last verified token.
//
// dflash2_select runs everything in ONE launch.  Every workgroup has up to
// two jobs, in this order:
//   * one slice of one H tile (the first n_proj workgroups); the last slice
//     of a tile to arrive sums the tile's slices;
//   * one contiguous vocabulary segment of one logits row (the first n_chunk
//     workgroups), streamed chunk by chunk, leaving a sorted list of K
//     candidates.
// Doing both in one workgroup keeps the grid small enough that segments do
// not queue for a free slot behind separate gate workgroups.
// Segment workgroups and summed H tiles then arrive on their sequence's
// counter (no workgroup ever waits for another).  The last to arrive
// finishes the sequence: it merges the rows' segment lists, scores the
// candidate pairs and walks the scores.
// Counters live in the scratch buffer and are reset by the workgroup that
// consumes them, so every launch starts from zero without a memset.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <utility>

#include "dflash2.h"
#include "common.hpp"
#include "finish.hpp"
#include "project.hpp"
#include "topk.hpp"

using namespace df2;

namespace {

// ----------------------------------------------------------------------------
// Launch description shared by the kernels (passed by value).
// ----------------------------------------------------------------------------
struct Params {
    const void* logits;
    const void* hidden;
    const void* A;
    const void* Bt;
    const void* W;
    const int32_t* prev;
    int32_t* out_path;
    float* out_score;
    // scratch
    uint64_t* part;       // [rows, nseg, K] candidate words
    int32_t* cand;        // [rows, K]
    float* cval;          // [rows, K]
    float* ppart;         // [S, M, r] gate partials
    float* H;             // [M, r]
    uint32_t* err;        // device input-error flags
    uint32_t* row_cnt;    // [rows]
    uint32_t* tile_cnt;   // [mtiles * qtiles]
    uint32_t* seq_cnt;    // [B]
    // sizes
    int B, P, V, d, r, K;
    int64_t rows;
    int C;                // chunks per row
    int nseg;             // segments per row
    int cps;              // chunks per segment
    int aligned;          // logits rows are 16-byte aligned and V % per-vector == 0
    int mtiles, qtiles, S, n_proj;
    int64_t n_chunk;      // segment workgroups (rows * nseg)
};

union SharedAll {
    ChunkLds c;
    ProjLds p;
    FinLds f;
};

__device__ __forceinline__ FinArgs fin_args(const Params& p) {
    FinArgs a;
    a.part = p.part;
    a.cand = nullptr;
    a.cval = nullptr;
    a.H = p.H;
    a.A = p.A;
    a.Bt = p.Bt;
    a.prev = p.prev;
    a.in_S = nullptr;
    a.in_cand = nullptr;
    a.out_S = nullptr;
    a.cand_out = p.cand;
    a.cval_out = p.cval;
    a.out_path = p.out_path;
    a.out_score = p.out_score;
    a.err = p.err;
    a.P = p.P;
    a.V = p.V;
    a.r = p.r;
    a.K = p.K;
    a.nseg = p.nseg;
    return a;
}

// Arrivals a sequence waits for: its P * nseg segments plus every H tile
// that covers one of its rows (one arrival per tile, once H is summed).
__device__ __forceinline__ uint32_t seq_expected(const Params& p, int b) {
    const int lo = b * p.P, hi = b * p.P + p.P - 1;
    const int n_mt = hi / 16 - lo / 16 + 1;
    return (uint32_t)(p.P * p.nseg + p.qtiles * n_mt);
}

// Arrival on the counters of sequences [b_lo, b_hi] (at most 16); returns
// the mask of those whose last arrival this was.  One thread per counter.
__device__ uint32_t arrive_seqs(const Params& p, int b_lo, int b_hi, uint32_t* flag) {
    drain_stores();
    __syncthreads();
    if (threadIdx.x < 64) {
        const int b = b_lo + (int)threadIdx.x;
        bool last = false;
        if (b <= b_hi) last = arrive(&p.seq_cnt[b]) == seq_expected(p, b) - 1u;
        const uint64_t bal = __ballot(last);
        if (threadIdx.x == 0) *flag = (uint32_t)bal;
    }
    __syncthreads();
    return *flag;
}

// A workgroup's role; returns a bit mask of the sequences (from *b0 on)
// whose finish falls to this workgroup (fused launches only).
template <bool BF16, int NV>
__device__ uint32_t chunk_role(const Params& p, int64_t sb, bool fused, SharedAll& sm,
                               uint32_t* flag, int* b0) {
    const int64_t row = sb / p.nseg;
    const int seg = (int)(sb % p.nseg);
    const size_t esz = BF16 ? 2 : 4;
    const char* rowp = reinterpret_cast<const char*>(p.logits) + (size_t)row * p.V * esz;
    const int c0 = seg * p.cps, c1 = min(p.C, c0 + p.cps);
    segment_topk<BF16, NV>(rowp, p.V, c0, c1, p.K, p.aligned != 0,
                           p.part + ((size_t)row * p.nseg + seg) * p.K, sm.c);
    if (!fused) {
        if (!block_arrive_last(&p.row_cnt[row], (uint32_t)p.nseg, flag)) return 0;
        merge_row<BF16>(p.part + (size_t)row * p.nseg * p.K, p.nseg, p.K, p.cand + row * p.K,
                        p.cval + row * p.K, sm.c);
        if (threadIdx.x == 0) reset_counter(&p.row_cnt[row]);
        return 0;
    }
    const int b = (int)(row / p.P);
    *b0 = b;
    return arrive_seqs(p, b, b, flag);
}

template <bool BF16, int NQ>
__device__ uint32_t proj_role(const Params& p, int pb, bool fused, SharedAll& sm, uint32_t* flag,
                              int* b0) {
    const int s = pb % p.S, tile = pb / p.S;
    const int mt = tile / p.qtiles, qt = tile % p.qtiles;
    const int M = (int)p.rows;
    proj_block<BF16, NQ>(p.hidden, p.W, M, p.d, p.r, mt, qt, s, p.S, p.S == 1 ? p.H : p.ppart,
                         sm.p);
    if (p.S > 1) {
        // the last slice of the tile to arrive sums the slices into H
        if (!block_arrive_last(&p.tile_cnt[tile], (uint32_t)p.S, flag)) return 0;
        proj_reduce_tile<NQ>(p.ppart, M, p.r, mt, qt, p.S, p.H);
        if (threadIdx.x == 0) reset_counter(&p.tile_cnt[tile]);
    }
    if (!fused) return 0;
    // a tile's 16 rows touch at most 16 sequences
    const int b_lo = (mt * 16) / p.P;
    const int b_hi = (min(M, mt * 16 + 16) - 1) / p.P;
    *b0 = b_lo;
    return arrive_seqs(p, b_lo, b_hi, flag);
}

// The whole selector in one launch.  Workgroup g computes H tile slice g
// first (g < n_proj; slice s of every tile lands on XCD s when there are
// eight slices, as workgroups are dealt to the XCDs round-robin), then
// streams segment g (g < n_chunk), then finishes the sequences whose last
// arrival it made.
template <bool BF16, int NV, int NQ>
__global__ __launch_bounds__(kWG, 5) void k_select(Params p) {
    __shared__ SharedAll sm;
    __shared__ uint32_t flag;
    const int64_t g = blockIdx.x;
    int pb0 = 0, cb0 = 0;
    uint32_t pmask = 0, cmask = 0;
    if (g < p.n_proj) pmask = proj_role<BF16, NQ>(p, (int)g, true, sm, &flag, &pb0);
    if (g < p.n_chunk) cmask = chunk_role<BF16, NV>(p, g, true, sm, &flag, &cb0);
    // a 16-bit gate mask and the segment's own sequence, in one word
    uint32_t mask = pmask | (cmask << 16);
    while (mask) {
        const int bit = __builtin_ctz(mask);
        mask &= mask - 1u;
        const int b = (bit < 16) ? pb0 + bit : cb0;
        finish_seq<BF16, kFinFused>(fin_args(p), b, sm.f);
        __syncthreads();
        if (threadIdx.x == 0) reset_counter(&p.seq_cnt[b]);
    }
}

// Top-K alone: chunk workgroups with the row merge on last arrival.
template <bool BF16, int NV>
__global__ __launch_bounds__(kWG, 5) void k_topk(Params p) {
    __shared__ SharedAll sm;
    __shared__ uint32_t flag;
    int b0 = 0;
    chunk_role<BF16, NV>(p, blockIdx.x, false, sm, &flag, &b0);
}

// Gate projection alone.
template <bool BF16, int NQ>
__global__ __launch_bounds__(kWG, 5) void k_project(Params p) {
    __shared__ SharedAll sm;
    __shared__ uint32_t flag;
    int b0 = 0;
    proj_role<BF16, NQ>(p, blockIdx.x, false, sm, &flag, &b0);
}

// Pair scores alone (written to global memory), or the walk alone.
template <bool BF16, int mode>
__global__ __launch_bounds__(kWG, 5) void k_finish(FinArgs a) {
    __shared__ FinLds sm;
    finish_seq<BF16, mode>(a, blockIdx.x, sm);
}

// ----------------------------------------------------------------------------
// Host side.
// ----------------------------------------------------------------------------
thread_local std::string g_last_error;

df2_status fail(df2_status s, const std::string& msg) {
    g_last_error = msg;
    return s;
}

df2_status hip_fail(hipError_t e, const char* what) {
    return fail(DF2_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

struct Scratch {
    void* ptr = nullptr;
    size_t bytes = 0;
    size_t zeroed_counter_bytes = 0;   // prefix known to hold only zeros
};

std::mutex g_mu;
std::map<std::pair<int, hipStream_t>, Scratch> g_scratch;

// Scratch of at least `bytes`, whose first `counter_bytes` are zero when the
// stream reaches the next launch.
df2_status get_scratch(hipStream_t stream, size_t bytes, size_t counter_bytes, void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    std::lock_guard<std::mutex> lock(g_mu);
    Scratch& s = g_scratch[std::make_pair(dev, stream)];
    if (s.bytes < bytes) {
        if (s.ptr) {
            e = hipStreamSynchronize(stream);
            if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
            (void)hipFree(s.ptr);
            s.ptr = nullptr;
            s.bytes = 0;
        }
        size_t nb = align_up(std::max(bytes, (size_t)1 << 20), (size_t)1 << 20);
        e = hipMalloc(&s.ptr, nb);
        if (e != hipSuccess) {
            s.ptr = nullptr;
            return fail(DF2_ENOMEM, std::string("hipMalloc scratch: ") + hipGetErrorString(e));
        }
        e = hipMemset(s.ptr, 0, nb);
        if (e != hipSuccess) return hip_fail(e, "hipMemset scratch");
        s.bytes = nb;
        s.zeroed_counter_bytes = nb;
    }
    if (s.zeroed_counter_bytes < counter_bytes) {
        e = hipMemsetAsync(s.ptr, 0, counter_bytes, stream);
        if (e != hipSuccess) return hip_fail(e, "hipMemsetAsync counters");
        s.zeroed_counter_bytes = counter_bytes;
    }
    *out = s.ptr;
    return DF2_OK;
}

// Later layouts may put data where earlier ones kept counters: remember that
// only the counter prefix of the latest layout is known to be zero.
void note_layout(hipStream_t stream, size_t counter_bytes) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return;
    std::lock_guard<std::mutex> lock(g_mu);
    auto it = g_scratch.find(std::make_pair(dev, stream));
    if (it != g_scratch.end()) it->second.zeroed_counter_bytes = counter_bytes;
}

int env_int(const char* name, int dflt) {
    const char* v = getenv(name);
    return (v && *v) ? atoi(v) : dflt;
}

struct Plan {
    Params p;
    int nv = 1, nq = 1;
    bool bf16 = true;
    int64_t n_chunk_blocks = 0;
    size_t counter_bytes = 0, total_bytes = 0;
    size_t off_part = 0, off_cand = 0, off_cval = 0, off_ppart = 0, off_H = 0;
};

// Chunk size (16-byte vectors per thread) and segmentation of the rows.
// Chunks of 256 x 4 vectors keep two register buffers per thread cheap;
// smaller chunks are used when there are too few rows to give every CU a
// workgroup.  Rows are then cut into segments so that about `target`
// workgroups stream in total, each pays one hand-off per segment, and the
// row merge stays within one workgroup's registers.
void plan_topk(Plan& pl, int64_t rows, int V, int K, bool bf16, const void* logits) {
    Params& p = pl.p;
    pl.bf16 = bf16;
    const int pv = bf16 ? 8 : 4;
    auto chunks = [&](int nv) { return (int)((V + (int64_t)kWG * pv * nv - 1) / ((int64_t)kWG * pv * nv)); };
    int nv = 1;
    for (int cand : {4, 2, 1}) {
        if (rows * chunks(cand) >= 256) { nv = cand; break; }
    }
    const int forced = env_int("DF2_NV", 0);
    if (forced == 1 || forced == 2 || forced == 4) nv = forced;
    pl.nv = nv;
    p.C = chunks(nv);
    const int64_t target = std::max(1, env_int("DF2_WGS", 1024));
    int nseg = (int)std::min<int64_t>(p.C, std::max<int64_t>(1, (target + rows - 1) / rows));
    int cps = (p.C + nseg - 1) / nseg;
    nseg = (p.C + cps - 1) / cps;
    while ((int64_t)nseg * K > kMergeMax) {
        ++cps;
        nseg = (p.C + cps - 1) / cps;
    }
    p.nseg = nseg;
    p.cps = cps;
    p.rows = rows;
    p.V = V;
    p.K = K;
    p.aligned = (aligned16(logits) && (V % pv) == 0) ? 1 : 0;
    pl.n_chunk_blocks = rows * nseg;
    p.n_chunk = pl.n_chunk_blocks;
}

// H tiles of 16 rows x 16*NQ columns, each cut into S slices of d (at most
// eight; eight puts slice s of every tile on XCD s).  Preferred: every wave
// issues all loads of its slice at once (one round trip), then the fewest
// slices; and, inside a select launch, no more slices than segment
// workgroups to host them.
void plan_proj(Plan& pl, int64_t M, int d, int r, int64_t hosts) {
    Params& p = pl.p;
    const int KS = d / 32;
    p.mtiles = (int)((M + 15) / 16);
    int best_nq = 1, best_S = 1;
    int64_t best_key = -1;
    for (int nq : {4, 2, 1}) {
        const int kb = proj_kb(pl.bf16, nq);
        int S = std::min(kMaxSlices, std::max(1, (KS + 4 * kb - 1) / (4 * kb)));
        S = std::min(S, KS);
        const int per_wave = ((KS + S - 1) / S + kWaves - 1) / kWaves;
        const int64_t batches = (per_wave + kb - 1) / kb;
        const int64_t n = (int64_t)p.mtiles * (r / (16 * nq)) * S;
        const bool fits = hosts <= 0 || n <= std::max<int64_t>(hosts, 256);
        const int64_t key = (fits ? 0 : (int64_t)1 << 40) + (batches << 24) + n;
        if (best_key < 0 || key < best_key) {
            best_key = key;
            best_nq = nq;
            best_S = S;
        }
    }
    int forced_nq = env_int("DF2_NQ", 0);
    if (forced_nq == 1 || forced_nq == 2 || forced_nq == 4) best_nq = forced_nq;
    int forced_s = env_int("DF2_S", 0);
    if (forced_s >= 1 && forced_s <= std::min(KS, kMaxSlices)) best_S = forced_s;
    pl.nq = best_nq;
    p.qtiles = r / (16 * pl.nq);
    p.S = best_S;
    p.n_proj = p.mtiles * p.qtiles * p.S;
    p.d = d;
    p.r = r;
}

// Scratch layout: counters first (err, row arrivals, tiles, sequences), then
// data.
void plan_layout(Plan& pl, int64_t rows, int64_t M, int B) {
    Params& p = pl.p;
    const size_t ncnt = 1 + (size_t)rows + (size_t)p.mtiles * p.qtiles + (size_t)B;
    pl.counter_bytes = align_up(ncnt * 4, 256);
    size_t off = pl.counter_bytes;
    pl.off_part = off;
    off = align_up(off + (size_t)rows * p.nseg * p.K * 8, 256);
    pl.off_cand = off;
    off = align_up(off + (size_t)rows * p.K * 4, 256);
    pl.off_cval = off;
    off = align_up(off + (size_t)rows * p.K * 4, 256);
    pl.off_ppart = off;
    off = align_up(off + (size_t)p.S * M * p.r * 4, 256);
    pl.off_H = off;
    off = align_up(off + (size_t)M * p.r * 4, 256);
    pl.total_bytes = off;
}

void bind_scratch(Plan& pl, void* base, int64_t rows, int B) {
    Params& p = pl.p;
    char* c = reinterpret_cast<char*>(base);
    uint32_t* cnt = reinterpret_cast<uint32_t*>(c);
    p.err = cnt;
    p.row_cnt = cnt + 1;
    p.tile_cnt = cnt + 1 + rows;
    p.seq_cnt = cnt + 1 + rows + (size_t)p.mtiles * p.qtiles;
    (void)B;
    p.part = reinterpret_cast<uint64_t*>(c + pl.off_part);
    p.cand = reinterpret_cast<int32_t*>(c + pl.off_cand);
    p.cval = reinterpret_cast<float*>(c + pl.off_cval);
    p.ppart = reinterpret_cast<float*>(c + pl.off_ppart);
    p.H = reinterpret_cast<float*>(c + pl.off_H);
}

df2_status check_dims(const df2_dims* dims, bool need_d) {
    if (!dims) return fail(DF2_EINVAL, "dims is NULL");
    if (dims->dtype != DF2_F32 && dims->dtype != DF2_BF16) return fail(DF2_EINVAL, "unknown dtype");
    if (dims->B < 0) return fail(DF2_EINVAL, "B < 0");
    if (dims->P < 1 || dims->P > kMaxP) return fail(DF2_EINVAL, "P must be in [1, 64]");
    if (dims->V < 1) return fail(DF2_EINVAL, "V < 1");
    if (need_d && (dims->d < 32 || dims->d % 32 != 0))
        return fail(DF2_EUNSUPPORTED, "d must be a positive multiple of 32");
    if (dims->r < 64 || dims->r % 64 != 0 || dims->r > kMaxR)
        return fail(DF2_EUNSUPPORTED, "r must be a multiple of 64 in [64, 512]");
    return DF2_OK;
}

df2_status check_k(int K, int V) {
    if (K < 1 || K > kMaxK || K > V) return fail(DF2_EINVAL, "K must be in [1, min(V, 64)]");
    return DF2_OK;
}

template <typename F>
df2_status launch_checked(F&& f, const char* what) {
    f();
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, what);
    return DF2_OK;
}

#define DF2_NV_CASES(BF, NQ_)                                                        \
    switch (pl.nv) {                                                                 \
        case 1: hipLaunchKernelGGL((k_select<BF, 1, NQ_>), grid, block, 0, stream, pl.p); break; \
        case 2: hipLaunchKernelGGL((k_select<BF, 2, NQ_>), grid, block, 0, stream, pl.p); break; \
        default: hipLaunchKernelGGL((k_select<BF, 4, NQ_>), grid, block, 0, stream, pl.p); break; \
    }

void launch_select(const Plan& pl, hipStream_t stream) {
    dim3 grid((unsigned)std::max<int64_t>(pl.p.n_proj, pl.n_chunk_blocks)), block(kWG);
    if (pl.bf16) {
        if (pl.nq == 4) { DF2_NV_CASES(true, 4) }
        else if (pl.nq == 2) { DF2_NV_CASES(true, 2) }
        else { DF2_NV_CASES(true, 1) }
    } else {
        if (pl.nq == 4) { DF2_NV_CASES(false, 4) }
        else if (pl.nq == 2) { DF2_NV_CASES(false, 2) }
        else { DF2_NV_CASES(false, 1) }
    }
}

void launch_topk(const Plan& pl, hipStream_t stream) {
    dim3 grid((unsigned)pl.n_chunk_blocks), block(kWG);
#define DF2_TOPK(BF)                                                                          \
    switch (pl.nv) {                                                                          \
        case 1: hipLaunchKernelGGL((k_topk<BF, 1>), grid, block, 0, stream, pl.p); break;   \
        case 2: hipLaunchKernelGGL((k_topk<BF, 2>), grid, block, 0, stream, pl.p); break;   \
        default: hipLaunchKernelGGL((k_topk<BF, 4>), grid, block, 0, stream, pl.p); break;  \
    }
    if (pl.bf16) { DF2_TOPK(true) } else { DF2_TOPK(false) }
#undef DF2_TOPK
}

void launch_project(const Plan& pl, hipStream_t stream) {
    dim3 grid((unsigned)pl.p.n_proj), block(kWG);
#define DF2_PROJ(BF)                                                                            \
    switch (pl.nq) {                                                                            \
        case 4: hipLaunchKernelGGL((k_project<BF, 4>), grid, block, 0, stream, pl.p); break;   \
        case 2: hipLaunchKernelGGL((k_project<BF, 2>), grid, block, 0, stream, pl.p); break;   \
        default: hipLaunchKernelGGL((k_project<BF, 1>), grid, block, 0, stream, pl.p); break;  \
    }
    if (pl.bf16) { DF2_PROJ(true) } else { DF2_PROJ(false) }
#undef DF2_PROJ
}

}  // namespace

// ----------------------------------------------------------------------------
// C ABI
// ----------------------------------------------------------------------------
extern "C" {

const char* dflash2_version(void) { return "0.1.0"; }

const char* dflash2_status_string(df2_status s) {
    switch (s) {
        case DF2_OK: return "ok";
        case DF2_EINVAL: return "invalid argument";
        case DF2_EUNSUPPORTED: return "unsupported argument";
        case DF2_EHIP: return "HIP error";
        case DF2_ENOMEM: return "out of device memory";
    }
    return "unknown status";
}

const char* dflash2_last_error(void) { return g_last_error.c_str(); }

df2_status dflash2_select(const df2_dims* dims, const void* logits, const void* hidden,
                          const void* A_tab, const void* B_tab, const void* W_H,
                          const int32_t* prev_tok, int32_t K, int32_t* out_path,
                          float* out_score, hipStream_t stream) {
    g_last_error.clear();
    df2_status st = check_dims(dims, true);
    if (st != DF2_OK) return st;
    if ((st = check_k(K, dims->V)) != DF2_OK) return st;
    if (dims->B == 0) return DF2_OK;
    if (!logits || !hidden || !A_tab || !B_tab || !W_H || !prev_tok || !out_path || !out_score)
        return fail(DF2_EINVAL, "NULL pointer argument");
    if (!aligned16(hidden) || !aligned16(A_tab) || !aligned16(B_tab) || !aligned16(W_H))
        return fail(DF2_EINVAL, "hidden, A_tab, B_tab and W_H must be 16-byte aligned");
    if (((uintptr_t)prev_tok & 3u) || ((uintptr_t)out_path & 3u) || ((uintptr_t)out_score & 3u))
        return fail(DF2_EINVAL, "prev_tok, out_path and out_score must be 4-byte aligned");
    const bool bf16 = dims->dtype == DF2_BF16;
    if (!bf16 && ((uintptr_t)logits & 3u)) return fail(DF2_EINVAL, "fp32 logits must be 4-byte aligned");
    if (bf16 && ((uintptr_t)logits & 1u)) return fail(DF2_EINVAL, "bf16 logits must be 2-byte aligned");
    const int64_t rows = (int64_t)dims->B * dims->P;
    Plan pl;
    std::memset(&pl.p, 0, sizeof(pl.p));
    plan_topk(pl, rows, dims->V, K, bf16, logits);
    plan_proj(pl, rows, dims->d, dims->r, pl.n_chunk_blocks);
    plan_layout(pl, rows, rows, dims->B);
    Params& p = pl.p;
    p.logits = logits;
    p.hidden = hidden;
    p.A = A_tab;
    p.Bt = B_tab;
    p.W = W_H;
    p.prev = prev_tok;
    p.out_path = out_path;
    p.out_score = out_score;
    p.B = dims->B;
    p.P = dims->P;
    void* base = nullptr;
    if ((st = get_scratch(stream, pl.total_bytes, pl.counter_bytes, &base)) != DF2_OK) return st;
    note_layout(stream, pl.counter_bytes);
    bind_scratch(pl, base, rows, dims->B);
    return launch_checked([&] { launch_select(pl, stream); }, "dflash2_select launch");
}

df2_status dflash2_topk(const void* logits, int64_t rows, int32_t V, df2_dtype dtype, int32_t K,
                        int32_t* out_idx, float* out_val, hipStream_t stream) {
    g_last_error.clear();
    if (dtype != DF2_F32 && dtype != DF2_BF16) return fail(DF2_EINVAL, "unknown dtype");
    if (rows < 0) return fail(DF2_EINVAL, "rows < 0");
    if (V < 1) return fail(DF2_EINVAL, "V < 1");
    df2_status st = check_k(K, V);
    if (st != DF2_OK) return st;
    if (rows == 0) return DF2_OK;
    if (!logits || !out_idx || !out_val) return fail(DF2_EINVAL, "NULL pointer argument");
    const bool bf16 = dtype == DF2_BF16;
    if (((uintptr_t)out_idx & 3u) || ((uintptr_t)out_val & 3u))
        return fail(DF2_EINVAL, "outputs must be 4-byte aligned");
    if ((bf16 && ((uintptr_t)logits & 1u)) || (!bf16 && ((uintptr_t)logits & 3u)))
        return fail(DF2_EINVAL, "logits misaligned for its dtype");
    Plan pl;
    std::memset(&pl.p, 0, sizeof(pl.p));
    plan_topk(pl, rows, V, K, bf16, logits);
    if (pl.n_chunk_blocks > 0x7FFFFFFF) return fail(DF2_EUNSUPPORTED, "too many rows");
    pl.p.mtiles = 0;
    pl.p.qtiles = 0;
    pl.p.S = 1;
    pl.p.r = 0;
    plan_layout(pl, rows, 0, 0);
    Params& p = pl.p;
    p.logits = logits;
    p.P = 1;
    void* base = nullptr;
    if ((st = get_scratch(stream, pl.total_bytes, pl.counter_bytes, &base)) != DF2_OK) return st;
    note_layout(stream, pl.counter_bytes);
    bind_scratch(pl, base, rows, 0);
    // results go straight to the caller's buffers
    p.cand = out_idx;
    p.cval = out_val;
    return launch_checked([&] { launch_topk(pl, stream); }, "dflash2_topk launch");
}

df2_status dflash2_project(const void* hidden, const void* W_H, int64_t M, int32_t d, int32_t r,
                           df2_dtype dtype, float* out_H, hipStream_t stream) {
    g_last_error.clear();
    if (dtype != DF2_F32 && dtype != DF2_BF16) return fail(DF2_EINVAL, "unknown dtype");
    if (M < 0) return fail(DF2_EINVAL, "M < 0");
    if (d < 32 || d % 32 != 0) return fail(DF2_EUNSUPPORTED, "d must be a positive multiple of 32");
    if (r < 64 || r % 64 != 0 || r > 1024)
        return fail(DF2_EUNSUPPORTED, "r must be a multiple of 64 in [64, 1024]");
    if (M == 0) return DF2_OK;
    if (M > (1 << 24)) return fail(DF2_EUNSUPPORTED, "M too large");
    if (!hidden || !W_H || !out_H) return fail(DF2_EINVAL, "NULL pointer argument");
    if (!aligned16(hidden) || !aligned16(W_H) || ((uintptr_t)out_H & 3u))
        return fail(DF2_EINVAL, "hidden and W_H must be 16-byte aligned, out_H 4-byte");
    Plan pl;
    std::memset(&pl.p, 0, sizeof(pl.p));
    pl.bf16 = dtype == DF2_BF16;
    plan_proj(pl, M, d, r, 0);
    pl.p.C = 0;
    pl.p.K = 0;
    plan_layout(pl, 0, M, 0);
    Params& p = pl.p;
    p.rows = M;
    p.hidden = hidden;
    p.W = W_H;
    void* base = nullptr;
    df2_status st;
    if ((st = get_scratch(stream, pl.total_bytes, pl.counter_bytes, &base)) != DF2_OK) return st;
    note_layout(stream, pl.counter_bytes);
    bind_scratch(pl, base, 0, 0);
    p.H = out_H;
    return launch_checked([&] { launch_project(pl, stream); }, "dflash2_project launch");
}

df2_status dflash2_pair_scores(const df2_dims* dims, const int32_t* cand_idx,
                               const float* cand_val, const float* H, const void* A_tab,
                               const void* B_tab, const int32_t* prev_tok, int32_t K,
                               float* out_S, hipStream_t stream) {
    g_last_error.clear();
    df2_status st = check_dims(dims, false);
    if (st != DF2_OK) return st;
    if ((st = check_k(K, dims->V)) != DF2_OK) return st;
    if (dims->B == 0) return DF2_OK;
    if (!cand_idx || !cand_val || !H || !A_tab || !B_tab || !prev_tok || !out_S)
        return fail(DF2_EINVAL, "NULL pointer argument");
    if (!aligned16(H) || !aligned16(A_tab) || !aligned16(B_tab))
        return fail(DF2_EINVAL, "H, A_tab and B_tab must be 16-byte aligned");
    void* base = nullptr;
    if ((st = get_scratch(stream, 256, 4, &base)) != DF2_OK) return st;
    FinArgs a;
    std::memset(&a, 0, sizeof(a));
    a.cand = cand_idx;
    a.cval = cand_val;
    a.H = H;
    a.A = A_tab;
    a.Bt = B_tab;
    a.prev = prev_tok;
    a.out_S = out_S;
    a.err = reinterpret_cast<uint32_t*>(base);
    a.P = dims->P;
    a.V = dims->V;
    a.r = dims->r;
    a.K = K;
    a.nseg = 1;
    dim3 grid((unsigned)dims->B), block(kWG);
    return launch_checked([&] {
        if (dims->dtype == DF2_BF16)
            hipLaunchKernelGGL((k_finish<true, kFinScores>), grid, block, 0, stream, a);
        else
            hipLaunchKernelGGL((k_finish<false, kFinScores>), grid, block, 0, stream, a);
    }, "dflash2_pair_scores launch");
}

df2_status dflash2_viterbi(const float* S, const int32_t* cand_idx, int32_t B, int32_t P,
                           int32_t K, int32_t* out_path, float* out_score, hipStream_t stream) {
    g_last_error.clear();
    if (B < 0) return fail(DF2_EINVAL, "B < 0");
    if (P < 1 || P > kMaxP) return fail(DF2_EINVAL, "P must be in [1, 64]");
    if (K < 1 || K > kMaxK) return fail(DF2_EINVAL, "K must be in [1, 64]");
    if (B == 0) return DF2_OK;
    if (!S || !cand_idx || !out_path || !out_score) return fail(DF2_EINVAL, "NULL pointer argument");
    FinArgs a;
    std::memset(&a, 0, sizeof(a));
    a.in_cand = cand_idx;
    a.in_S = S;
    a.out_path = out_path;
    a.out_score = out_score;
    a.P = P;
    a.K = K;
    a.r = 64;
    a.nseg = 1;
    a.V = 0x7FFFFFFF;
    dim3 grid((unsigned)B), block(kWG);
    return launch_checked([&] {
        hipLaunchKernelGGL((k_finish<true, kFinWalk>), grid, block, 0, stream, a);
    }, "dflash2_viterbi launch");
}

df2_status dflash2_device_error(hipStream_t stream, uint32_t* flags) {
    g_last_error.clear();
    if (!flags) return fail(DF2_EINVAL, "flags is NULL");
    *flags = 0;
    hipError_t e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
    int dev = 0;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return hip_fail(e, "hipGetDevice");
    void* ptr = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_mu);
        auto it = g_scratch.find(std::make_pair(dev, stream));
        if (it == g_scratch.end()) return DF2_OK;
        ptr = it->second.ptr;
    }
    uint32_t v = 0;
    if ((e = hipMemcpy(&v, ptr, 4, hipMemcpyDeviceToHost)) != hipSuccess) return hip_fail(e, "hipMemcpy flags");
    if (v) {
        const uint32_t zero = 0;
        if ((e = hipMemcpy(ptr, &zero, 4, hipMemcpyHostToDevice)) != hipSuccess)
            return hip_fail(e, "hipMemcpy flags");
    }
    *flags = v;
    return DF2_OK;
}

df2_status dflash2_release(void) {
    g_last_error.clear();
    std::lock_guard<std::mutex> lock(g_mu);
    df2_status st = DF2_OK;
    for (auto& kv : g_scratch) {
        if (!kv.second.ptr) continue;
        int cur = 0;
        (void)hipGetDevice(&cur);
        (void)hipSetDevice(kv.first.first);
        hipError_t e = hipFree(kv.second.ptr);
        (void)hipSetDevice(cur);
        if (e != hipSuccess) st = hip_fail(e, "hipFree");
    }
    g_scratch.clear();
    return st;
}

}  // extern "C"
