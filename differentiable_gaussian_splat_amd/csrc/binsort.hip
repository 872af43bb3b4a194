// Tile binning with a (tile, depth) key sort.
//
// Sorting the P (tile, Gaussian) pairs by the 64-bit key (tile << 32 | depth
// bits), equal keys by Gaussian index, gives each tile its Gaussians front to
// back. This file reaches exactly that order without sorting the P pairs
// (P is 44.5M for 1M Gaussians at 1920x1080):
//   1. stable compaction of the visible Gaussians (index order kept);
//   2. LSD radix sort of those N by their 32 depth bits (stable: equal depths
//      stay in index order), so the pair stream "each Gaussian's tiles, in
//      depth order" is the order every tile's list must follow;
//   3. exclusive scan of their tile counts in that order: each one's first
//      pair index;
//   4. chunked placement (below): per-tile counts of each chunk of the pair
//      stream, their prefix over chunks, and one wave per chunk writing every
//      pair to its final slot with per-tile LDS cursors.
// For tile grids too large for LDS cursors, a stable LSD radix sort of the
// generated pairs by tile id does step 4 instead.
// Radix passes rank stably with wave64 ballot matching against per-wave LDS
// counters (no barrier per round) and stage the block in LDS so that the
// output is written in contiguous runs. The pair count P is reduced first and
// copied to the host asynchronously, so the host's wait for it overlaps the
// depth sort.
#include "common.hpp"
#include "launch.hpp"

namespace gs {

namespace {

constexpr int SB = 256;       // threads per block
constexpr int SI = 16;        // scan items per thread
constexpr int ST = SB * SI;   // scan items per block

typedef unsigned long long u64;

__device__ __forceinline__ int eff_count(int n, const u64* dcount) {
    if (!dcount) return n;
    u64 c = *dcount;
    return c < (u64)n ? (int)c : n;
}

// Exclusive scan of one u32 per thread across the 256-thread block.
__device__ __forceinline__ uint32_t block_excl_scan_u32(uint32_t v, uint32_t* s_w, uint32_t& total) {
    int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    uint32_t x = v;
    for (int off = 1; off < 64; off <<= 1) {
        uint32_t y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    if (lane == 63) s_w[w] = x;
    __syncthreads();
    uint32_t pre = 0, tot = 0;
    for (int i = 0; i < SB / 64; ++i) {
        uint32_t t = s_w[i];
        pre += i < w ? t : 0u;
        tot += t;
    }
    __syncthreads();
    total = tot;
    return pre + x - v;
}

// Inclusive max-scan of one u32 per thread across the block.
__device__ __forceinline__ uint32_t block_incl_max_u32(uint32_t v, uint32_t* s_w) {
    int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    uint32_t x = v;
    for (int off = 1; off < 64; off <<= 1) {
        uint32_t y = __shfl_up(x, off);
        if (lane >= off) x = max(x, y);
    }
    if (lane == 63) s_w[w] = x;
    __syncthreads();
    for (int i = 0; i < w; ++i) x = max(x, s_w[i]);
    __syncthreads();
    return x;
}

// ---------------------------------------------------------------- scans

struct LoadPlain {
    const uint32_t* p;
    __device__ uint32_t operator()(int i) const { return p[i]; }
};
struct LoadVisible {
    const uint32_t* tiles;
    __device__ uint32_t operator()(int i) const { return tiles[i] > 0u ? 1u : 0u; }
};
struct LoadSortedTiles {
    const uint32_t* tiles;
    const uint32_t* order;
    __device__ uint32_t operator()(int i) const { return tiles[order[i]]; }
};
struct StoreInPlace {
    uint32_t* p;
    __device__ void operator()(int i, u64 pos, uint32_t) const { p[i] = (uint32_t)pos; }
};
struct StoreCompact {
    const float* depths;
    uint32_t* keys;
    uint32_t* idx;
    __device__ void operator()(int i, u64 pos, uint32_t flag) const {
        if (flag) {
            keys[pos] = __float_as_uint(depths[i]);
            idx[pos] = (uint32_t)i;
        }
    }
};
struct StoreRanges {
    uint2* ranges;
    __device__ void operator()(int t, u64 pos, uint32_t cnt) const {
        ranges[t] = cnt ? make_uint2((uint32_t)pos, (uint32_t)pos + cnt) : make_uint2(0u, 0u);
    }
};

// Block sums in 64 bits, so that a grand total beyond 2^32 is seen as such.
template <class Load>
__global__ __launch_bounds__(SB) void k_scan_reduce(Load ld, int n, const u64* dcount, u64* partials) {
    __shared__ u64 s_w[SB / 64];
    int cnt = eff_count(n, dcount);
    int base = blockIdx.x * ST;
    u64 sum = 0;
    for (int j = 0; j < SI; ++j) {
        int i = base + j * SB + threadIdx.x;
        if (i < cnt) sum += ld(i);
    }
    for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
    if ((threadIdx.x & 63) == 0) s_w[threadIdx.x >> 6] = sum;
    __syncthreads();
    if (threadIdx.x == 0) partials[blockIdx.x] = s_w[0] + s_w[1] + s_w[2] + s_w[3];
}

// One 1024-thread block: exclusive scan of the block partials in place; the
// grand total goes to *total.
__global__ __launch_bounds__(1024) void k_scan_top(u64* partials, int nb, u64* total) {
    __shared__ u64 s_w[16];
    int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    u64 carry = 0;
    for (int base = 0; base < nb; base += 1024) {
        int i = base + threadIdx.x;
        u64 v = i < nb ? partials[i] : 0ull;
        u64 x = v;
        for (int off = 1; off < 64; off <<= 1) {
            u64 y = __shfl_up(x, off);
            if (lane >= off) x += y;
        }
        if (lane == 63) s_w[w] = x;
        __syncthreads();
        u64 pre = 0, tot = 0;
        for (int k = 0; k < 16; ++k) {
            u64 t = s_w[k];
            pre += k < w ? t : 0ull;
            tot += t;
        }
        if (i < nb) partials[i] = carry + pre + x - v;
        carry += tot;
        __syncthreads();
    }
    if (threadIdx.x == 0 && total) *total = carry;
}

template <class Load, class Store>
__global__ __launch_bounds__(SB) void k_scan_down(Load ld, Store st, int n, const u64* dcount, const u64* partials) {
    __shared__ uint32_t s_val[ST];
    __shared__ uint32_t s_pre[ST];
    __shared__ uint32_t s_w[SB / 64];
    int cnt = eff_count(n, dcount);
    int base = blockIdx.x * ST;
    if (base >= cnt) return;
    for (int j = 0; j < SI; ++j) {
        int li = j * SB + threadIdx.x;
        int i = base + li;
        s_val[li] = i < cnt ? ld(i) : 0u;
    }
    __syncthreads();
    uint32_t local[SI];
    uint32_t sum = 0;
    for (int m = 0; m < SI; ++m) {
        local[m] = s_val[threadIdx.x * SI + m];
        sum += local[m];
    }
    uint32_t tot;
    uint32_t run = block_excl_scan_u32(sum, s_w, tot);
    for (int m = 0; m < SI; ++m) {
        s_pre[threadIdx.x * SI + m] = run;
        run += local[m];
    }
    __syncthreads();
    u64 boff = partials[blockIdx.x];
    for (int j = 0; j < SI; ++j) {
        int li = j * SB + threadIdx.x;
        int i = base + li;
        if (i < cnt) st(i, boff + s_pre[li], s_val[li]);
    }
}

__global__ __launch_bounds__(SB) void k_fill_u32(uint32_t* p, size_t count, uint32_t value) {
    size_t i = (size_t)blockIdx.x * SB + threadIdx.x;
    size_t stride = (size_t)gridDim.x * SB;
    for (; i < count; i += stride) p[i] = value;
}

hipError_t fill(uint32_t* p, size_t count, uint32_t value, hipStream_t s) {
    if (count == 0) return hipSuccess;
    size_t blocks = (count + SB - 1) / SB;
    if (blocks > 4096) blocks = 4096;
    k_fill_u32<<<(int)blocks, SB, 0, s>>>(p, count, value);
    return hipGetLastError();
}

// Grand total only (reduce + scan of partials).
template <class Load>
hipError_t reduce_total(Load ld, int n, u64* partials, u64* total, hipStream_t s) {
    int nb = (n + ST - 1) / ST;
    if (nb == 0) return fill(reinterpret_cast<uint32_t*>(total), 2, 0u, s);
    k_scan_reduce<Load><<<nb, SB, 0, s>>>(ld, n, nullptr, partials);
    k_scan_top<<<1, 1024, 0, s>>>(partials, nb, total);
    return hipGetLastError();
}

// Small arrays (n <= 16K): one 1024-thread block, each thread a contiguous run of <= 16.
template <class Load, class Store>
__global__ __launch_bounds__(1024) void k_scan_single(Load ld, Store st, int n, const u64* dcount, u64* total) {
    __shared__ u64 s_w[16];
    const int cnt = eff_count(n, dcount);
    const int per = (cnt + 1023) / 1024;
    const int b = threadIdx.x * per, e = min(cnt, b + per);
    u64 sum = 0;
    for (int i = b; i < e; ++i) sum += ld(i);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    u64 x = sum;
    for (int off = 1; off < 64; off <<= 1) {
        u64 y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    if (lane == 63) s_w[w] = x;
    __syncthreads();
    u64 pre = 0, tot = 0;
    for (int k = 0; k < 16; ++k) {
        pre += k < w ? s_w[k] : 0ull;
        tot += s_w[k];
    }
    u64 run = pre + x - sum;
    for (int i = b; i < e; ++i) {
        const uint32_t v = ld(i);
        st(i, run, v);
        run += v;
    }
    if (threadIdx.x == 0 && total) *total = tot;
}

template <class Load, class Store>
hipError_t scan(Load ld, Store st, int n, const u64* dcount, u64* partials, u64* total, hipStream_t s) {
    int nb = (n + ST - 1) / ST;
    if (nb == 0) return total ? fill(reinterpret_cast<uint32_t*>(total), 2, 0u, s) : hipSuccess;
    if (n <= 16384) {
        k_scan_single<Load, Store><<<1, 1024, 0, s>>>(ld, st, n, dcount, total);
        return hipGetLastError();
    }
    k_scan_reduce<Load><<<nb, SB, 0, s>>>(ld, n, dcount, partials);
    k_scan_top<<<1, 1024, 0, s>>>(partials, nb, total);
    k_scan_down<Load, Store><<<nb, SB, 0, s>>>(ld, st, n, dcount, partials);
    return hipGetLastError();
}

// ---------------------------------------------------------------- chunked tile binning
//
// The depth-ordered pair stream is cut into chunks at Gaussian boundaries
// (chunk c holds the Gaussians whose first pair index lies in [c CH, (c+1) CH)).
// k_chunk_counts counts each chunk's pairs per tile; a prefix over chunks gives
// each chunk, per tile, the number of that tile's pairs in earlier chunks; and
// k_chunk_place walks the chunk's Gaussians in depth order with one LDS cursor
// per tile, writing each pair straight to its final slot. The order within a
// tile is therefore chunk order, then depth order inside the chunk: the full
// (tile, depth, index) order, with no pass over the pairs besides the two that
// generate them.

__device__ __forceinline__ int lower_bound_u32(const uint32_t* a, int n, uint32_t x) {
    int lo = 0, hi = n;  // first index with a[i] >= x, n if none
    while (lo < hi) {
        int mid = (lo + hi) >> 1;
        if (a[mid] < x) lo = mid + 1; else hi = mid;
    }
    return lo;
}

// Up to 64 consecutive depth-sorted Gaussians staged by one wave, with the
// exclusive prefix of their tile counts: the batch's pairs are then walked
// 64 at a time ("windows"), whatever the Gaussians' sizes.
struct BatchLds {
    uint32_t g[64], rect[64], wd[64], pre[64], db[64], mark[64];
};

__device__ __forceinline__ uint32_t wave_excl_scan_u32(uint32_t v, uint32_t& total) {
    const int lane = threadIdx.x & 63;
    uint32_t x = v;
    for (int off = 1; off < 64; off <<= 1) {
        uint32_t y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    total = __shfl(x, 63);
    return x - v;
}

__device__ __forceinline__ uint32_t wave_incl_max_u32(uint32_t v) {
    const int lane = threadIdx.x & 63;
    for (int off = 1; off < 64; off <<= 1) {
        uint32_t y = __shfl_up(v, off);
        if (lane >= off) v = max(v, y);
    }
    return v;
}

// Stages Gaussians kb .. kb+nb-1 (all loads in flight at once); returns the batch's pair count.
__device__ __forceinline__ uint32_t load_batch(BatchLds& B, int kb, int nb, const uint32_t* __restrict__ order,
                                               const float2* __restrict__ means2d, const int* __restrict__ radii,
                                               const float* __restrict__ depths, int TX, int TY) {
    const int lane = threadIdx.x & 63;
    uint32_t nt = 0;
    wave_lds_sync();  // the previous batch's entries have been read
    if (lane < nb) {
        const uint32_t g = order[kb + lane];
        const float2 m = means2d[g];
        int X0, X1, Y0, Y1;
        tile_rect(m.x, m.y, radii[g], TX, TY, X0, X1, Y0, Y1);
        nt = (uint32_t)((X1 - X0 + 1) * (Y1 - Y0 + 1));
        B.g[lane] = g;
        B.rect[lane] = (uint32_t)X0 | ((uint32_t)Y0 << 16);
        B.wd[lane] = (uint32_t)(X1 - X0 + 1);
        B.db[lane] = depths ? __float_as_uint(depths[g]) : 0u;
    }
    uint32_t total;
    B.pre[lane] = wave_excl_scan_u32(nt, total);
    wave_lds_sync();  // batch_window reads other lanes' entries
    return total;
}

// Window of pairs f0 .. f0+63 of the batch: each lane's Gaussian (batch index)
// and tile. `cur` is the Gaussian covering f0; it advances to the one covering f0+63.
__device__ __forceinline__ void batch_window(BatchLds& B, int nb, uint32_t f0, uint32_t& cur, int TX, uint32_t& i,
                                             uint32_t& t) {
    const int lane = threadIdx.x & 63;
    wave_lds_sync();  // every lane has read the previous window's marks
    B.mark[lane] = 0u;
    wave_lds_sync();
    if (lane < nb) {
        const uint32_t st = B.pre[lane];
        if (st >= f0 && st < f0 + 64u) B.mark[st - f0] = (uint32_t)lane + 1u;  // one start per slot: counts >= 1
    }
    wave_lds_sync();  // slot `lane` may have been written by another lane
    const uint32_t m = wave_incl_max_u32(B.mark[lane]);
    i = m ? m - 1u : cur;
    cur = __shfl(i, 63);
    const int j = (int)(f0 + (uint32_t)lane - B.pre[i]);
    const int wd = (int)B.wd[i];
    int q, r;
    divmod_small(j, wd, q, r);
    const uint32_t rect = B.rect[i];
    t = (uint32_t)(((int)(rect >> 16) + q) * TX + (int)(rect & 0xffffu) + r);
}

__global__ __launch_bounds__(256) void k_chunk_counts(int CH, const u64* vis_ptr, const uint32_t* __restrict__ offsets,
                                                    const uint32_t* __restrict__ order,
                                                    const float2* __restrict__ means2d, const int* __restrict__ radii,
                                                    int TX, int TY, uint32_t* __restrict__ counts) {
    extern __shared__ uint32_t s_cnt[];
    __shared__ BatchLds s_b[SB / 64];
    __shared__ int s_k[2];
    const int ntiles = TX * TY;
    const int c = blockIdx.x;
    for (int t = threadIdx.x; t < ntiles; t += SB) s_cnt[t] = 0u;
    if (threadIdx.x == 0) {
        const int vis = (int)*vis_ptr;
        s_k[0] = lower_bound_u32(offsets, vis, (uint32_t)c * (uint32_t)CH);
        s_k[1] = lower_bound_u32(offsets, vis, (uint32_t)(c + 1) * (uint32_t)CH);
    }
    __syncthreads();
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    BatchLds& B = s_b[w];
    // the waves take batches in turn; counting needs no order
    for (int kb = s_k[0] + 64 * w; kb < s_k[1]; kb += 64 * (SB / 64)) {
        const int nb = min(64, s_k[1] - kb);
        const uint32_t T = load_batch(B, kb, nb, order, means2d, radii, nullptr, TX, TY);
        uint32_t cur = 0;
        for (uint32_t f0 = 0; f0 < T; f0 += 64u) {
            uint32_t i, t;
            batch_window(B, nb, f0, cur, TX, i, t);
            if (f0 + (uint32_t)lane < T && t < (uint32_t)ntiles) atomicAdd(&s_cnt[t], 1u);
        }
    }
    __syncthreads();
    uint32_t* row = counts + (size_t)c * ntiles;
    for (int t = threadIdx.x; t < ntiles; t += SB) row[t] = s_cnt[t];
}

// Per tile: segment sums of the chunk counts (segments of SEG chunks).
__global__ __launch_bounds__(SB) void k_seg_sum(int nchunks, int ntiles, int SEG, const uint32_t* __restrict__ counts,
                                              uint32_t* __restrict__ segsum) {
    const int nseg = (nchunks + SEG - 1) / SEG;
    const int idx = blockIdx.x * SB + threadIdx.x;
    if (idx >= nseg * ntiles) return;
    const int sg = idx / ntiles, t = idx - sg * ntiles;
    const int c1 = min(nchunks, (sg + 1) * SEG);
    uint32_t acc = 0;
    for (int c = sg * SEG; c < c1; ++c) acc += counts[(size_t)c * ntiles + t];
    segsum[idx] = acc;
}

// Per tile: exclusive scan over segments (in place) and the tile's total.
__global__ __launch_bounds__(SB) void k_seg_scan(int nseg, int ntiles, uint32_t* __restrict__ segsum,
                                               uint32_t* __restrict__ total) {
    const int t = blockIdx.x * SB + threadIdx.x;
    if (t >= ntiles) return;
    uint32_t run = 0;
    for (int sg = 0; sg < nseg; ++sg) {
        const uint32_t v = segsum[(size_t)sg * ntiles + t];
        segsum[(size_t)sg * ntiles + t] = run;
        run += v;
    }
    total[t] = run;
}

// Per (segment, tile): running prefix over the segment's chunks, turning the
// counts in place into each chunk's per-tile base.
__global__ __launch_bounds__(SB) void k_chunk_base(int nchunks, int ntiles, int SEG, uint32_t* __restrict__ counts,
                                                 const uint32_t* __restrict__ segbase) {
    const int nseg = (nchunks + SEG - 1) / SEG;
    const int idx = blockIdx.x * SB + threadIdx.x;
    if (idx >= nseg * ntiles) return;
    const int sg = idx / ntiles, t = idx - sg * ntiles;
    const int c1 = min(nchunks, (sg + 1) * SEG);
    uint32_t run = segbase[idx];
    for (int c = sg * SEG; c < c1; ++c) {
        const uint32_t v = counts[(size_t)c * ntiles + t];
        counts[(size_t)c * ntiles + t] = run;
        run += v;
    }
}

// One wave per chunk: stable placement with per-tile LDS cursors. Each window
// of 64 pairs ranks lanes with equal tiles by ballot matching (lanes are in
// depth order), so the cursor of a tile advances in depth order.
__global__ __launch_bounds__(64) void k_chunk_place(int CH, const u64* vis_ptr, const uint32_t* __restrict__ offsets,
                                                  const uint32_t* __restrict__ order,
                                                  const float2* __restrict__ means2d, const int* __restrict__ radii,
                                                  const float* __restrict__ depths, int TX, int TY, int tbits, int P,
                                                  const uint32_t* __restrict__ base, const uint2* __restrict__ ranges,
                                                  uint32_t* __restrict__ values, u64* __restrict__ keys64) {
    extern __shared__ uint32_t s_cur[];
    __shared__ BatchLds B;
    const int ntiles = TX * TY;
    const int c = blockIdx.x;
    const int lane = threadIdx.x;
    const int vis = (int)*vis_ptr;
    const int k0 = lower_bound_u32(offsets, vis, (uint32_t)c * (uint32_t)CH);
    const int k1 = lower_bound_u32(offsets, vis, (uint32_t)(c + 1) * (uint32_t)CH);
    const uint32_t* row = base + (size_t)c * ntiles;
    for (int t = lane; t < ntiles; t += 64) s_cur[t] = ranges[t].x + row[t];
    __syncthreads();
    const uint64_t lt = lanemask_lt();
    for (int kb = k0; kb < k1; kb += 64) {
        const int nb = min(64, k1 - kb);
        const uint32_t T = load_batch(B, kb, nb, order, means2d, radii, keys64 ? depths : nullptr, TX, TY);
        uint32_t cur = 0;
        for (uint32_t f0 = 0; f0 < T; f0 += 64u) {
            uint32_t i, t;
            batch_window(B, nb, f0, cur, TX, i, t);
            // a pair always lies inside the grid and its tile's range; the
            // check only keeps a broken invariant from writing out of bounds
            const bool valid = f0 + (uint32_t)lane < T && t < (uint32_t)ntiles;
            uint64_t peers = __ballot(valid);
            for (int bb = 0; bb < tbits; ++bb) {
                const bool bit = (t >> bb) & 1u;
                const uint64_t m = __ballot(bit);
                peers &= bit ? m : ~m;
            }
            if (valid) {
                const uint32_t lrank = (uint32_t)__popcll(peers & lt);
                const uint32_t b0 = s_cur[t];
                const uint32_t pos = b0 + lrank;
                if (lrank == 0u) s_cur[t] = b0 + (uint32_t)__popcll(peers);
                const uint32_t g = B.g[i];
                if (pos < (uint32_t)P) {
                    values[pos] = g;
                    if (keys64) keys64[pos] = ((u64)t << 32) | (u64)B.db[i];
                }
            }
            wave_lds_sync();  // cursor updates seen by the next window
        }
    }
}

// ---------------------------------------------------------------- radix sort

// Keys and values read from memory.
struct SrcMem {
    static constexpr int E = 4096;          // elements per block
    static constexpr int LDS_WORDS = 0;
    const uint32_t* keys;
    const uint32_t* vals;
    __device__ void setup(int, int, uint32_t*) const {}
    __device__ uint32_t key(int p, const uint32_t*, int) const { return keys[p]; }
    __device__ void get(int p, uint32_t& k, uint32_t& v, const uint32_t*, int) const {
        k = keys[p];
        v = vals[p];
    }
};

// (tile, Gaussian) pairs generated in depth order: pair p belongs to the
// depth-sorted Gaussian k with offsets[k] <= p < offsets[k+1] and is the
// (p - offsets[k])-th tile of its rectangle in row-major order.
struct SrcPairs {
    static constexpr int E = 2048;
    // gid, off, g, rect, width (E each), k0 and nk, per-thread maxima (SB), per-wave maxima
    static constexpr int LDS_WORDS = 5 * E + 2 + SB + SB / 64;
    const uint32_t* offsets;
    const uint32_t* order;
    const float2* means2d;
    const int* radii;
    const u64* vis;
    int TX, TY;

    __device__ void setup(int p0, int p1, uint32_t* lds) const {
        uint32_t* s_gid = lds;
        uint32_t* s_off = lds + E;
        uint32_t* s_g = lds + 2 * E;
        uint32_t* s_rect = lds + 3 * E;
        uint32_t* s_wd = lds + 4 * E;
        uint32_t* s_k = lds + 5 * E;
        if (threadIdx.x == 0) {
            int nvis = (int)*vis;
            int k0 = 0, nk = 0;
            if (p0 < p1 && nvis > 0) {
                // largest k with offsets[k] <= p, for p = p0 and p = p1 - 1
                int lo = 0, hi = nvis - 1;
                while (lo < hi) {
                    int mid = (lo + hi + 1) >> 1;
                    if ((int)offsets[mid] <= p0) lo = mid; else hi = mid - 1;
                }
                k0 = lo;
                hi = nvis - 1;
                while (lo < hi) {
                    int mid = (lo + hi + 1) >> 1;
                    if ((int)offsets[mid] <= p1 - 1) lo = mid; else hi = mid - 1;
                }
                nk = lo - k0 + 1;  // <= p1 - p0: every visible Gaussian owns >= 1 pair
            }
            s_k[0] = (uint32_t)k0;
            s_k[1] = (uint32_t)nk;
        }
        for (int e = threadIdx.x; e < E; e += SB) s_gid[e] = 0u;
        __syncthreads();
        const int k0 = (int)s_k[0], nk = (int)s_k[1];
        for (int i = threadIdx.x; i < nk; i += SB) {
            uint32_t g = order[k0 + i];
            float2 m = means2d[g];
            int X0, X1, Y0, Y1;
            tile_rect(m.x, m.y, radii[g], TX, TY, X0, X1, Y0, Y1);
            uint32_t off = offsets[k0 + i];
            s_off[i] = off;
            s_g[i] = g;
            s_rect[i] = (uint32_t)X0 | ((uint32_t)Y0 << 16);
            s_wd[i] = (uint32_t)(X1 - X0 + 1);
            int e = (int)off - p0;
            if (e > 0 && e < E) s_gid[e] = (uint32_t)i;  // Gaussian i starts at block element e
        }
        __syncthreads();
        // prefix-max of the start markers: element e belongs to the last Gaussian starting at or before it
        constexpr int R = E / SB;
        uint32_t* s_tmax = lds + 5 * E + 2;
        uint32_t* s_w = lds + 5 * E + 2 + SB;
        uint32_t loc[R];
        uint32_t m = 0;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            m = max(m, s_gid[threadIdx.x * R + r]);
            loc[r] = m;
        }
        s_tmax[threadIdx.x] = block_incl_max_u32(m, s_w);
        __syncthreads();
        const uint32_t excl = threadIdx.x > 0 ? s_tmax[threadIdx.x - 1] : 0u;
#pragma unroll
        for (int r = 0; r < R; ++r) s_gid[threadIdx.x * R + r] = max(loc[r], excl);
        __syncthreads();
    }

    __device__ void decode(int p, const uint32_t* lds, int p0, uint32_t& tile, uint32_t& g) const {
        const uint32_t i = lds[p - p0];
        const int j = p - (int)lds[E + i];
        const int wdt = (int)lds[4 * E + i];
        const uint32_t rect = lds[3 * E + i];
        // q = j / wdt, r = j % wdt via a float reciprocal and one exact fixup
        int q = (int)(((float)j + 0.5f) * __builtin_amdgcn_rcpf((float)wdt));
        int rr = j - q * wdt;
        if (rr < 0) { q -= 1; rr += wdt; }
        if (rr >= wdt) { q += 1; rr -= wdt; }
        tile = (uint32_t)(((int)(rect >> 16) + q) * TX + (int)(rect & 0xffffu) + rr);
        g = lds[2 * E + i];
    }
    __device__ uint32_t key(int p, const uint32_t* lds, int p0) const {
        uint32_t t, g;
        decode(p, lds, p0, t, g);
        return t;
    }
    __device__ void get(int p, uint32_t& k, uint32_t& v, const uint32_t* lds, int p0) const { decode(p, lds, p0, k, v); }
};

template <class Src>
__global__ __launch_bounds__(SB) void k_ms_hist(Src src, int n, const u64* dcount, int shift, int bits, int nblocks,
                                              uint32_t* __restrict__ hist) {
    constexpr int E = Src::E, R = E / SB;
    __shared__ uint32_t lds[Src::LDS_WORDS > 0 ? Src::LDS_WORDS : 1];
    __shared__ uint32_t s_h[4][256];
    for (int k = threadIdx.x; k < 4 * 256; k += SB) (&s_h[0][0])[k] = 0u;
    const int cnt = eff_count(n, dcount);
    const int p0 = blockIdx.x * E;
    const int p1 = min(cnt, p0 + E);
    src.setup(p0, p1, lds);
    __syncthreads();
    const uint32_t mask = (1u << bits) - 1u;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll 4
    for (int r = 0; r < R; ++r) {
        int p = p0 + w * R * 64 + r * 64 + lane;
        if (p < p1) atomicAdd(&s_h[w][(src.key(p, lds, p0) >> shift) & mask], 1u);
    }
    __syncthreads();
    const int nbins = 1 << bits;
    if ((int)threadIdx.x < nbins)
        hist[(size_t)threadIdx.x * nblocks + blockIdx.x] =
            s_h[0][threadIdx.x] + s_h[1][threadIdx.x] + s_h[2][threadIdx.x] + s_h[3][threadIdx.x];
}

// Stable scatter of one radix digit. Wave w owns the block's elements
// [w E/4, (w+1) E/4) in rounds of 64 consecutive ones; within a round, lanes
// with equal digits are matched by ballots and ranked against the wave's own
// LDS counters (no barrier per round); after one barrier the per-digit wave
// offsets are combined, the block is reordered in LDS by (digit, rank), and
// written out so that each digit's elements form one contiguous run.
template <class Src>
__global__ __launch_bounds__(SB) void k_ms_scatter(Src src, int n, const u64* dcount, int shift, int bits,
                                                 int nblocks, const uint32_t* __restrict__ hist_scanned,
                                                 uint32_t* __restrict__ keys_out, uint32_t* __restrict__ vals_out,
                                                 u64* __restrict__ keys64_out, const float* __restrict__ depths) {
    constexpr int E = Src::E, R = E / SB;
    constexpr int LW = Src::LDS_WORDS > 2 * E ? Src::LDS_WORDS : 2 * E;
    __shared__ uint32_t lds[LW];  // the source's staging, later the output staging
    __shared__ uint32_t s_wcnt[4][256];
    __shared__ uint32_t s_wpre[4][256];
    __shared__ uint32_t s_dstart[256];
    __shared__ uint32_t s_gbase[256];
    __shared__ uint32_t s_w[SB / 64];
    const int cnt = eff_count(n, dcount);
    const int p0 = blockIdx.x * E;
    if (p0 >= cnt) return;
    const int p1 = min(cnt, p0 + E);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int nbins = 1 << bits;
    const uint32_t mask = (uint32_t)nbins - 1u;
    src.setup(p0, p1, lds);
    for (int k = lane; k < 256; k += 64) s_wcnt[w][k] = 0u;
    wave_lds_sync();
    s_gbase[tid] = tid < nbins ? hist_scanned[(size_t)tid * nblocks + blockIdx.x] : 0u;
    uint32_t kk[R], vv[R], rk[R];
    const int ebase = p0 + w * R * 64 + lane;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        int p = ebase + r * 64;
        kk[r] = 0u;
        vv[r] = 0u;
        if (p < p1) src.get(p, kk[r], vv[r], lds, p0);
    }
    const uint64_t lt = lanemask_lt();
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const bool valid = ebase + r * 64 < p1;
        const uint32_t d = (kk[r] >> shift) & mask;
        uint64_t peers = __ballot(valid);
        for (int b = 0; b < bits; ++b) {
            const bool bit = (d >> b) & 1u;
            const uint64_t bb = __ballot(bit);
            peers &= bit ? bb : ~bb;
        }
        const uint32_t lrank = (uint32_t)__popcll(peers & lt);
        const uint32_t base = s_wcnt[w][d];
        rk[r] = base + lrank;
        if (valid && lrank == 0u) s_wcnt[w][d] = base + (uint32_t)__popcll(peers);
        wave_lds_sync();  // the wave's counters are read by other lanes next round
    }
    __syncthreads();
    uint32_t c0 = 0, c1 = 0, c2 = 0;
    uint32_t tot = 0;
    if (tid < nbins) {
        c0 = s_wcnt[0][tid];
        c1 = s_wcnt[1][tid];
        c2 = s_wcnt[2][tid];
        tot = c0 + c1 + c2 + s_wcnt[3][tid];
    }
    uint32_t all;
    const uint32_t ds = block_excl_scan_u32(tot, s_w, all);
    if (tid < nbins) {
        s_dstart[tid] = ds;
        s_wpre[0][tid] = ds;
        s_wpre[1][tid] = ds + c0;
        s_wpre[2][tid] = ds + c0 + c1;
        s_wpre[3][tid] = ds + c0 + c1 + c2;
    }
    __syncthreads();
    uint32_t* s_keys = lds;
    uint32_t* s_vals = lds + E;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if (ebase + r * 64 < p1) {
            const uint32_t slot = s_wpre[w][(kk[r] >> shift) & mask] + rk[r];
            s_keys[slot] = kk[r];
            s_vals[slot] = vv[r];
        }
    }
    __syncthreads();
    const int here = p1 - p0;
    for (int sl = tid; sl < here; sl += SB) {
        const uint32_t key = s_keys[sl];
        const uint32_t val = s_vals[sl];
        const uint32_t d = (key >> shift) & mask;
        const uint32_t dst = s_gbase[d] + ((uint32_t)sl - s_dstart[d]);
        if (keys_out) keys_out[dst] = key;
        vals_out[dst] = val;
        if (keys64_out) keys64_out[dst] = ((u64)key << 32) | (u64)__float_as_uint(depths[val]);
    }
}

template <class Src>
hipError_t radix_pass(Src src, int n, const u64* dcount, int shift, int bits, uint32_t* hist, u64* partials,
                      uint32_t* keys_out, uint32_t* vals_out, u64* keys64_out, const float* depths, hipStream_t s) {
    const int nblocks = (n + Src::E - 1) / Src::E;
    if (nblocks == 0) return hipSuccess;
    k_ms_hist<Src><<<nblocks, SB, 0, s>>>(src, n, dcount, shift, bits, nblocks, hist);
    hipError_t e = scan(LoadPlain{hist}, StoreInPlace{hist}, (1 << bits) * nblocks, nullptr, partials, nullptr, s);
    if (e != hipSuccess) return e;
    k_ms_scatter<Src><<<nblocks, SB, 0, s>>>(src, n, dcount, shift, bits, nblocks, hist, keys_out, vals_out, keys64_out,
                                             depths);
    return hipGetLastError();
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int bits_for(int ntiles) {
    int b = 1;
    while ((1 << b) < ntiles) ++b;
    return b;
}

// Ranges from tile-sorted keys (radix path only).
__global__ __launch_bounds__(SB) void k_ranges(int P, const uint32_t* __restrict__ tile_keys, uint2* __restrict__ ranges) {
    int p = blockIdx.x * SB + threadIdx.x;
    if (p >= P) return;
    uint32_t t = tile_keys[p];
    if (p == 0 || tile_keys[p - 1] != t) ranges[t].x = (uint32_t)p;
    if (p == P - 1 || tile_keys[p + 1] != t) ranges[t].y = (uint32_t)(p + 1);
}

constexpr int MAX_CHUNK_TILES = 14336;  // LDS cursors or counters of one chunk: 56 KB, plus the staged batches under 64 KB
constexpr int MAX_CHUNKS = 2048;
constexpr int MIN_CHUNK_PAIRS = 8192;
constexpr int SEG = 32;                  // chunks per segment of the prefix over chunks

}  // namespace

hipError_t launch_fill_u32(uint32_t* p, size_t count, uint32_t value, hipStream_t stream) {
    return fill(p, count, value, stream);
}

BinLayout bin_layout(int64_t n, int64_t capacity, int TX, int TY) {
    BinLayout L;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off += align256(bytes);
        return o;
    };
    size_t nn = (size_t)(n > 0 ? n : 1), cap = (size_t)(capacity > 0 ? capacity : 1);
    size_t ntiles = (size_t)TX * TY;
    const bool chunked = ntiles <= (size_t)MAX_CHUNK_TILES;
    L.dkeys[0] = take(4 * nn);
    L.dkeys[1] = take(4 * nn);
    L.didx[0] = take(4 * nn);
    L.didx[1] = take(4 * nn);
    L.offsets = take(4 * (nn + 1));
    size_t hist_entries = 256 * ((nn + SrcMem::E - 1) / SrcMem::E);
    if (!chunked) {
        size_t hp = 256 * ((cap + SrcPairs::E - 1) / SrcPairs::E);
        if (hp > hist_entries) hist_entries = hp;
    }
    size_t max_scan = hist_entries;
    if (nn > max_scan) max_scan = nn;
    if (ntiles > max_scan) max_scan = ntiles;
    L.partials = take(8 * ((max_scan + ST - 1) / ST + 1));
    L.hist = take(4 * hist_entries);
    L.counters = take(8 * 4);
    if (chunked) {
        L.chunk_counts = take(4 * (size_t)MAX_CHUNKS * ntiles);
        L.seg = take(4 * (size_t)((MAX_CHUNKS + SEG - 1) / SEG) * ntiles);
        L.tile_total = take(4 * ntiles);
        L.tkeys[0] = L.tkeys[1] = L.tvals = 0;
    } else {
        L.chunk_counts = L.seg = L.tile_total = 0;
        L.tkeys[0] = take(4 * cap);
        L.tkeys[1] = take(4 * cap);
        L.tvals = take(4 * cap);
    }
    L.total = off;
    return L;
}

hipError_t launch_bin_count(int n, const float* depths, const uint32_t* tiles_touched, char* ws, const BinLayout& L,
                            unsigned long long* host_P, hipEvent_t ev, hipStream_t s) {
    u64* counters = reinterpret_cast<u64*>(ws + L.counters);
    u64* partials = reinterpret_cast<u64*>(ws + L.partials);
    hipError_t e = fill(reinterpret_cast<uint32_t*>(counters), 8, 0u, s);
    if (e != hipSuccess) return e;
    // the pair count first, on its way to the host while the rest runs
    e = reduce_total(LoadPlain{tiles_touched}, n, partials, &counters[2], s);
    if (e == hipSuccess) e = hipMemcpyAsync(host_P, &counters[2], sizeof(u64), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipEventRecord(ev, s);
    if (e != hipSuccess || n == 0) return e;
    uint32_t* dk[2] = {reinterpret_cast<uint32_t*>(ws + L.dkeys[0]), reinterpret_cast<uint32_t*>(ws + L.dkeys[1])};
    uint32_t* di[2] = {reinterpret_cast<uint32_t*>(ws + L.didx[0]), reinterpret_cast<uint32_t*>(ws + L.didx[1])};
    // 1. visible compaction (index order kept): depth bits and indices
    e = scan(LoadVisible{tiles_touched}, StoreCompact{depths, dk[0], di[0]}, n, nullptr, partials, &counters[0], s);
    if (e != hipSuccess) return e;
    // 2. stable sort by the 32 depth bits, 4 passes of 8: the result returns to buffer 0
    uint32_t* hist = reinterpret_cast<uint32_t*>(ws + L.hist);
    for (int pass = 0; pass < 4; ++pass) {
        int c = pass & 1;
        e = radix_pass(SrcMem{dk[c], di[c]}, n, &counters[0], 8 * pass, 8, hist, partials, dk[c ^ 1], di[c ^ 1],
                       nullptr, nullptr, s);
        if (e != hipSuccess) return e;
    }
    // 3. first pair index of each depth-sorted Gaussian
    uint32_t* offsets = reinterpret_cast<uint32_t*>(ws + L.offsets);
    return scan(LoadSortedTiles{tiles_touched, di[0]}, StoreInPlace{offsets}, n, &counters[0], partials, &counters[1],
                s);
}

hipError_t launch_bin_emit(int n, int P, int TX, int TY, const float* means2d, const int* radii, const float* depths,
                           char* ws, const BinLayout& L, uint64_t* keys, uint32_t* values, uint32_t* ranges,
                           hipStream_t s) {
    const int ntiles = TX * TY;
    u64* counters = reinterpret_cast<u64*>(ws + L.counters);
    u64* partials = reinterpret_cast<u64*>(ws + L.partials);
    const uint32_t* offsets = reinterpret_cast<const uint32_t*>(ws + L.offsets);
    const uint32_t* order = reinterpret_cast<const uint32_t*>(ws + L.didx[0]);
    const float2* m2 = reinterpret_cast<const float2*>(means2d);
    u64* k64 = reinterpret_cast<u64*>(keys);
    if (P == 0 || n == 0) return fill(ranges, (size_t)2 * ntiles, 0u, s);

    if (ntiles <= MAX_CHUNK_TILES) {
        const int CH = max(MIN_CHUNK_PAIRS, (P + MAX_CHUNKS - 1) / MAX_CHUNKS);
        const int nchunks = (P + CH - 1) / CH;
        const int nseg = (nchunks + SEG - 1) / SEG;
        uint32_t* counts = reinterpret_cast<uint32_t*>(ws + L.chunk_counts);
        uint32_t* seg = reinterpret_cast<uint32_t*>(ws + L.seg);
        uint32_t* total = reinterpret_cast<uint32_t*>(ws + L.tile_total);
        const size_t lds = sizeof(uint32_t) * ntiles;
        k_chunk_counts<<<nchunks, 256, lds, s>>>(CH, &counters[0], offsets, order, m2, radii, TX, TY, counts);
        const int nst = nseg * ntiles;
        k_seg_sum<<<(nst + SB - 1) / SB, SB, 0, s>>>(nchunks, ntiles, SEG, counts, seg);
        k_seg_scan<<<(ntiles + SB - 1) / SB, SB, 0, s>>>(nseg, ntiles, seg, total);
        hipError_t e = scan(LoadPlain{total}, StoreRanges{reinterpret_cast<uint2*>(ranges)}, ntiles, nullptr, partials,
                            nullptr, s);
        if (e != hipSuccess) return e;
        k_chunk_base<<<(nst + SB - 1) / SB, SB, 0, s>>>(nchunks, ntiles, SEG, counts, seg);
        k_chunk_place<<<nchunks, 64, lds, s>>>(CH, &counters[0], offsets, order, m2, radii, depths, TX, TY,
                                               bits_for(ntiles), P, counts, reinterpret_cast<const uint2*>(ranges),
                                               values, k64);
        return hipGetLastError();
    }

    // large tile grids: stable LSD radix sort of the generated pairs by tile id
    hipError_t e = fill(ranges, (size_t)2 * ntiles, 0u, s);
    if (e != hipSuccess) return e;
    uint32_t* hist = reinterpret_cast<uint32_t*>(ws + L.hist);
    uint32_t* tk[2] = {reinterpret_cast<uint32_t*>(ws + L.tkeys[0]), reinterpret_cast<uint32_t*>(ws + L.tkeys[1])};
    uint32_t* tv = reinterpret_cast<uint32_t*>(ws + L.tvals);
    const int tbits = bits_for(ntiles);
    const int passes = (tbits + 7) / 8;
    const int bpp = (tbits + passes - 1) / passes;
    SrcPairs gen{offsets, order, m2, radii, &counters[0], TX, TY};
    // value buffers alternate so that the last pass writes `values` (pass i
    // writes `values` when passes - 1 - i is even); tile keys alternate in tk
    uint32_t* kin = nullptr;
    uint32_t* vin = nullptr;
    for (int pass = 0; pass < passes; ++pass) {
        const int shift = pass * bpp;
        const int bits = min(bpp, tbits - shift);
        const bool last = pass == passes - 1;
        uint32_t* kout = tk[pass & 1];
        uint32_t* vout = ((passes - 1 - pass) % 2 == 0) ? values : tv;
        u64* k64out = last ? k64 : nullptr;
        if (pass == 0)
            e = radix_pass(gen, P, nullptr, shift, bits, hist, partials, kout, vout, k64out, depths, s);
        else
            e = radix_pass(SrcMem{kin, vin}, P, nullptr, shift, bits, hist, partials, kout, vout, k64out, depths, s);
        if (e != hipSuccess) return e;
        kin = kout;
        vin = vout;
    }
    k_ranges<<<(P + SB - 1) / SB, SB, 0, s>>>(P, kin, reinterpret_cast<uint2*>(ranges));
    return hipGetLastError();
}

}  // namespace gs
