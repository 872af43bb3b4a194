// Tile binning with a (tile, depth) key sort.
//
// Sorting P pairs by the 64-bit key (tile << 32 | depth bits) and then by
// Gaussian index gives each tile its Gaussians front to back. This file reaches
// the same order in fewer passes over the P pairs:
//   1. compact the visible Gaussians (stable, so index order is kept);
//   2. LSD radix-sort them by the 32 depth bits (stable: equal depths stay in
//      index order) -- N elements instead of P;
//   3. exclusive scan of their tile counts in that order gives each one's
//      pair offset and the total P;
//   4. emit the pairs in depth order, one thread per pair (load balanced:
//      each thread finds its Gaussian by binary search over the offsets);
//   5. stable LSD radix sort of the pairs by tile id only
//      (ceil(log2 #tiles) bits: 13 at 1920x1080, two passes). Stability keeps
//      the depth order inside each tile, so the result equals the full-key sort.
//   6. per-tile [first, last) ranges; optionally the 64-bit keys.
// Every scan and radix pass is a three-kernel reduce / scan-of-partials /
// down-sweep over blocks of 4096 elements; sorts are stable within a block via
// wave64 ballot matching.
#include "common.hpp"
#include "launch.hpp"

namespace gs {

namespace {

constexpr int SB = 256;       // threads per block
constexpr int SI = 16;        // items per thread
constexpr int ST = SB * SI;   // items per block
constexpr int DUP = 2048;     // pairs per block in the emission kernel

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

template <class Load>
__global__ __launch_bounds__(SB) void k_scan_reduce(Load ld, int n, const u64* dcount, u64* partials) {
    __shared__ uint32_t s_w[SB / 64];
    int cnt = eff_count(n, dcount);
    int base = blockIdx.x * ST;
    uint32_t sum = 0;
    for (int j = 0; j < SI; ++j) {
        int i = base + j * SB + threadIdx.x;
        if (i < cnt) sum += ld(i);
    }
    uint32_t tot;
    block_excl_scan_u32(sum, s_w, tot);
    if (threadIdx.x == 0) partials[blockIdx.x] = tot;
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

template <class Load, class Store>
hipError_t scan(Load ld, Store st, int n, const u64* dcount, u64* partials, u64* total, hipStream_t s) {
    int nb = (n + ST - 1) / ST;
    if (nb == 0) {
        if (total) k_fill_u32<<<1, SB, 0, s>>>(reinterpret_cast<uint32_t*>(total), 2, 0u);
        return hipGetLastError();
    }
    k_scan_reduce<Load><<<nb, SB, 0, s>>>(ld, n, dcount, partials);
    k_scan_top<<<1, 1024, 0, s>>>(partials, nb, total);
    k_scan_down<Load, Store><<<nb, SB, 0, s>>>(ld, st, n, dcount, partials);
    return hipGetLastError();
}

// ---------------------------------------------------------------- radix sort

__global__ __launch_bounds__(SB) void k_radix_hist(const uint32_t* __restrict__ keys, int n, const u64* dcount,
                                                 int shift, int bits, int nblocks, uint32_t* __restrict__ hist) {
    __shared__ uint32_t s_h[4][256];
    for (int k = threadIdx.x; k < 4 * 256; k += SB) (&s_h[0][0])[k] = 0u;
    __syncthreads();
    int cnt = eff_count(n, dcount);
    int base = blockIdx.x * ST;
    uint32_t mask = (1u << bits) - 1u;
    int w = threadIdx.x >> 6;
    for (int j = 0; j < SI; ++j) {
        int i = base + j * SB + threadIdx.x;
        if (i < cnt) atomicAdd(&s_h[w][(keys[i] >> shift) & mask], 1u);
    }
    __syncthreads();
    int nbins = 1 << bits;
    if ((int)threadIdx.x < nbins)
        hist[(size_t)threadIdx.x * nblocks + blockIdx.x] =
            s_h[0][threadIdx.x] + s_h[1][threadIdx.x] + s_h[2][threadIdx.x] + s_h[3][threadIdx.x];
}

// Stable scatter of one radix digit. Ranks inside the block follow element
// order: per 256-element round, lanes with equal digits are matched by wave
// ballots, counts are combined across the 4 waves in LDS, and a running count
// per digit carries across rounds. The block's elements are then reordered
// in LDS by (digit, rank) and written out so that equal digits form
// contiguous runs in the output.
__global__ __launch_bounds__(SB) void k_radix_scatter(const uint32_t* __restrict__ keys_in,
                                                    const uint32_t* __restrict__ vals_in,
                                                    uint32_t* __restrict__ keys_out, uint32_t* __restrict__ vals_out,
                                                    int n, const u64* dcount, int shift, int bits, int nblocks,
                                                    const uint32_t* __restrict__ hist_scanned) {
    __shared__ uint32_t s_keys[ST];
    __shared__ uint32_t s_vals[ST];
    __shared__ uint32_t s_cnt[4][256];
    __shared__ uint32_t s_pre[4][256];
    __shared__ uint32_t s_dstart[256];
    __shared__ uint32_t s_gbase[256];
    __shared__ uint32_t s_w[SB / 64];
    int cnt = eff_count(n, dcount);
    int base = blockIdx.x * ST;
    if (base >= cnt) return;
    int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    int nbins = 1 << bits;
    uint32_t mask = (uint32_t)nbins - 1u;
    for (int k = tid; k < 4 * 256; k += SB) (&s_cnt[0][0])[k] = 0u;
    s_gbase[tid] = tid < nbins ? hist_scanned[(size_t)tid * nblocks + blockIdx.x] : 0u;
    uint32_t kk[SI], vv[SI], rk[SI];
    for (int j = 0; j < SI; ++j) {
        int i = base + j * SB + tid;
        bool valid = i < cnt;
        kk[j] = valid ? keys_in[i] : 0u;
        vv[j] = valid ? vals_in[i] : 0u;
    }
    __syncthreads();
    uint32_t run = 0;  // thread tid keeps the running count of digit tid
    uint64_t lt = lanemask_lt();
    for (int j = 0; j < SI; ++j) {
        int i = base + j * SB + tid;
        bool valid = i < cnt;
        uint32_t d = (kk[j] >> shift) & mask;
        uint64_t peers = __ballot(valid);
        for (int b = 0; b < bits; ++b) {
            bool bit = (d >> b) & 1u;
            uint64_t bb = __ballot(bit);
            peers &= bit ? bb : ~bb;
        }
        uint32_t lrank = (uint32_t)__popcll(peers & lt);
        if (valid && lrank == 0u) s_cnt[w][d] = (uint32_t)__popcll(peers);
        __syncthreads();
        if (tid < nbins) {
            uint32_t c0 = s_cnt[0][tid], c1 = s_cnt[1][tid], c2 = s_cnt[2][tid], c3 = s_cnt[3][tid];
            s_cnt[0][tid] = 0u;
            s_cnt[1][tid] = 0u;
            s_cnt[2][tid] = 0u;
            s_cnt[3][tid] = 0u;
            s_pre[0][tid] = run;
            s_pre[1][tid] = run + c0;
            s_pre[2][tid] = run + c0 + c1;
            s_pre[3][tid] = run + c0 + c1 + c2;
            run += c0 + c1 + c2 + c3;
        }
        __syncthreads();
        rk[j] = valid ? s_pre[w][d] + lrank : 0u;
    }
    uint32_t tot;
    uint32_t ds = block_excl_scan_u32(tid < nbins ? run : 0u, s_w, tot);
    s_dstart[tid] = ds;
    __syncthreads();
    for (int j = 0; j < SI; ++j) {
        int i = base + j * SB + tid;
        if (i < cnt) {
            uint32_t d = (kk[j] >> shift) & mask;
            uint32_t slot = s_dstart[d] + rk[j];
            s_keys[slot] = kk[j];
            s_vals[slot] = vv[j];
        }
    }
    __syncthreads();
    int here = min(ST, cnt - base);
    for (int j = 0; j < SI; ++j) {
        int sl = j * SB + tid;
        if (sl < here) {
            uint32_t key = s_keys[sl];
            uint32_t d = (key >> shift) & mask;
            uint32_t dst = s_gbase[d] + ((uint32_t)sl - s_dstart[d]);
            keys_out[dst] = key;
            vals_out[dst] = s_vals[sl];
        }
    }
}

// Sorts (k[0], v[0]) by `total_bits` low key bits using (k[1], v[1]) as the
// second buffer; returns the index (0 or 1) of the buffer holding the result.
int radix_sort(uint32_t* k[2], uint32_t* v[2], int n, const u64* dcount, int total_bits, uint32_t* hist,
               u64* partials, hipStream_t s, hipError_t& err) {
    int passes = (total_bits + 7) / 8;
    int bpp = (total_bits + passes - 1) / passes;
    int nblocks = (n + ST - 1) / ST;
    int cur = 0;
    err = hipSuccess;
    if (nblocks == 0) return 0;
    for (int p = 0; p < passes; ++p) {
        int shift = p * bpp;
        int bits = min(bpp, total_bits - shift);
        k_radix_hist<<<nblocks, SB, 0, s>>>(k[cur], n, dcount, shift, bits, nblocks, hist);
        int nh = (1 << bits) * nblocks;
        err = scan(LoadPlain{hist}, StoreInPlace{hist}, nh, nullptr, partials, nullptr, s);
        if (err != hipSuccess) return cur;
        k_radix_scatter<<<nblocks, SB, 0, s>>>(k[cur], v[cur], k[cur ^ 1], v[cur ^ 1], n, dcount, shift, bits,
                                               nblocks, hist);
        cur ^= 1;
    }
    err = hipGetLastError();
    return cur;
}

// ---------------------------------------------------------------- pairs

// One thread per pair. The block's pair range [p0, p1) spans the sorted
// Gaussians k0..k1; their offsets and tile rectangles are staged in LDS, and
// each thread finds its Gaussian by binary search there.
__global__ __launch_bounds__(SB) void k_emit_pairs(int P, int vis, const uint32_t* __restrict__ offsets,
                                                 const uint32_t* __restrict__ order, const float2* __restrict__ means2d,
                                                 const int* __restrict__ radii, int TX, int TY,
                                                 uint32_t* __restrict__ tile_keys, uint32_t* __restrict__ values) {
    __shared__ uint32_t s_off[DUP];
    __shared__ uint32_t s_g[DUP];
    __shared__ int s_x0[DUP], s_w[DUP], s_y0[DUP];
    __shared__ int s_k0, s_nk;
    int p0 = blockIdx.x * DUP;
    int p1 = min(P, p0 + DUP);
    if (threadIdx.x == 0) {
        // largest k with offsets[k] <= p, for p = p0 and p = p1 - 1
        int lo = 0, hi = vis - 1;
        while (lo < hi) {
            int mid = (lo + hi + 1) >> 1;
            if ((int)offsets[mid] <= p0) lo = mid; else hi = mid - 1;
        }
        int k0 = lo;
        hi = vis - 1;
        while (lo < hi) {
            int mid = (lo + hi + 1) >> 1;
            if ((int)offsets[mid] <= p1 - 1) lo = mid; else hi = mid - 1;
        }
        s_k0 = k0;
        s_nk = lo - k0 + 1;
    }
    __syncthreads();
    int k0 = s_k0, nk = s_nk;
    for (int i = threadIdx.x; i < nk; i += SB) {
        uint32_t g = order[k0 + i];
        float2 m = means2d[g];
        int X0, X1, Y0, Y1;
        tile_rect(m.x, m.y, radii[g], TX, TY, X0, X1, Y0, Y1);
        s_off[i] = offsets[k0 + i];
        s_g[i] = g;
        s_x0[i] = X0;
        s_w[i] = X1 - X0 + 1;
        s_y0[i] = Y0;
    }
    __syncthreads();
    for (int p = p0 + threadIdx.x; p < p1; p += SB) {
        int lo = 0, hi = nk - 1;
        while (lo < hi) {
            int mid = (lo + hi + 1) >> 1;
            if ((int)s_off[mid] <= p) lo = mid; else hi = mid - 1;
        }
        int j = p - (int)s_off[lo];
        int wdt = s_w[lo];
        int ty = s_y0[lo] + j / wdt;
        int tx = s_x0[lo] + j % wdt;
        tile_keys[p] = (uint32_t)(ty * TX + tx);
        values[p] = s_g[lo];
    }
}

__global__ __launch_bounds__(SB) void k_ranges(int P, const uint32_t* __restrict__ tile_keys, uint2* __restrict__ ranges) {
    int p = blockIdx.x * SB + threadIdx.x;
    if (p >= P) return;
    uint32_t t = tile_keys[p];
    if (p == 0 || tile_keys[p - 1] != t) ranges[t].x = (uint32_t)p;
    if (p == P - 1 || tile_keys[p + 1] != t) ranges[t].y = (uint32_t)(p + 1);
}

__global__ __launch_bounds__(SB) void k_keys64(int P, const uint32_t* __restrict__ tile_keys,
                                             const uint32_t* __restrict__ values, const float* __restrict__ depths,
                                             u64* __restrict__ keys) {
    int p = blockIdx.x * SB + threadIdx.x;
    if (p >= P) return;
    keys[p] = ((u64)tile_keys[p] << 32) | (u64)__float_as_uint(depths[values[p]]);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int bits_for(int ntiles) {
    int b = 1;
    while ((1 << b) < ntiles) ++b;
    return b;
}

}  // namespace

hipError_t launch_fill_u32(uint32_t* p, size_t count, uint32_t value, hipStream_t stream) {
    if (count == 0) return hipSuccess;
    size_t blocks = (count + SB - 1) / SB;
    if (blocks > 4096) blocks = 4096;
    k_fill_u32<<<(int)blocks, SB, 0, stream>>>(p, count, value);
    return hipGetLastError();
}

BinLayout bin_layout(int64_t n, int64_t capacity, int ntiles) {
    BinLayout L;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off += align256(bytes);
        return o;
    };
    size_t nn = (size_t)(n > 0 ? n : 1), cap = (size_t)(capacity > 0 ? capacity : 1);
    L.dkeys[0] = take(4 * nn);
    L.dkeys[1] = take(4 * nn);
    L.didx[0] = take(4 * nn);
    L.didx[1] = take(4 * nn);
    L.offsets = take(4 * (nn + 1));
    size_t maxel = nn > cap ? nn : cap;
    size_t nblocks = (maxel + ST - 1) / ST;
    size_t hist_entries = 256 * nblocks;
    size_t max_scan = hist_entries > maxel ? hist_entries : maxel;
    L.partials = take(8 * ((max_scan + ST - 1) / ST + 1));
    L.hist = take(4 * hist_entries);
    L.counters = take(8 * 4);
    L.tkeys[0] = take(4 * cap);
    L.tkeys[1] = take(4 * cap);
    L.tvals = take(4 * cap);
    (void)ntiles;
    L.total = off;
    return L;
}

hipError_t launch_bin_count(int n, const float* depths, const uint32_t* tiles_touched, char* ws,
                            const BinLayout& L, hipStream_t s) {
    u64* counters = reinterpret_cast<u64*>(ws + L.counters);
    hipError_t e = launch_fill_u32(reinterpret_cast<uint32_t*>(counters), 8, 0u, s);
    if (e != hipSuccess || n == 0) return e;
    u64* partials = reinterpret_cast<u64*>(ws + L.partials);
    uint32_t* dk[2] = {reinterpret_cast<uint32_t*>(ws + L.dkeys[0]), reinterpret_cast<uint32_t*>(ws + L.dkeys[1])};
    uint32_t* di[2] = {reinterpret_cast<uint32_t*>(ws + L.didx[0]), reinterpret_cast<uint32_t*>(ws + L.didx[1])};
    // 1. visible compaction (index order kept): depth bits and indices
    e = scan(LoadVisible{tiles_touched}, StoreCompact{depths, dk[0], di[0]}, n, nullptr, partials, &counters[0], s);
    if (e != hipSuccess) return e;
    // 2. stable sort by depth bits
    uint32_t* hist = reinterpret_cast<uint32_t*>(ws + L.hist);
    int cur = radix_sort(dk, di, n, &counters[0], 32, hist, partials, s, e);
    if (e != hipSuccess) return e;
    if (cur != 0) return hipErrorUnknown;  // 4 passes always end in buffer 0
    // 3. pair offsets in depth order and the total P
    uint32_t* offsets = reinterpret_cast<uint32_t*>(ws + L.offsets);
    e = scan(LoadSortedTiles{tiles_touched, di[0]}, StoreInPlace{offsets}, n, &counters[0], partials, &counters[1], s);
    return e;
}

hipError_t launch_bin_emit(int n, int vis, int P, int TX, int TY, const float* means2d, const int* radii,
                           const float* depths, char* ws, const BinLayout& L, uint64_t* keys, uint32_t* values,
                           uint32_t* ranges, hipStream_t s) {
    int ntiles = TX * TY;
    hipError_t e = launch_fill_u32(ranges, (size_t)2 * ntiles, 0u, s);
    if (e != hipSuccess || P == 0) return e;
    (void)n;
    u64* partials = reinterpret_cast<u64*>(ws + L.partials);
    uint32_t* offsets = reinterpret_cast<uint32_t*>(ws + L.offsets);
    uint32_t* order = reinterpret_cast<uint32_t*>(ws + L.didx[0]);
    uint32_t* hist = reinterpret_cast<uint32_t*>(ws + L.hist);
    int tbits = bits_for(ntiles);
    int passes = (tbits + 7) / 8;
    // the last radix pass must land in `values`
    uint32_t* tk[2] = {reinterpret_cast<uint32_t*>(ws + L.tkeys[0]), reinterpret_cast<uint32_t*>(ws + L.tkeys[1])};
    uint32_t* tv[2];
    if (passes % 2 == 0) {
        tv[0] = values;
        tv[1] = reinterpret_cast<uint32_t*>(ws + L.tvals);
    } else {
        tv[0] = reinterpret_cast<uint32_t*>(ws + L.tvals);
        tv[1] = values;
    }
    int blocks = (P + DUP - 1) / DUP;
    k_emit_pairs<<<blocks, SB, 0, s>>>(P, vis, offsets, order, reinterpret_cast<const float2*>(means2d), radii, TX,
                                       TY, tk[0], tv[0]);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    int cur = radix_sort(tk, tv, P, nullptr, tbits, hist, partials, s, e);
    if (e != hipSuccess) return e;
    if (tv[cur] != values) return hipErrorUnknown;
    int pb = (P + SB - 1) / SB;
    k_ranges<<<pb, SB, 0, s>>>(P, tk[cur], reinterpret_cast<uint2*>(ranges));
    if (keys) k_keys64<<<pb, SB, 0, s>>>(P, tk[cur], values, depths, reinterpret_cast<u64*>(keys));
    return hipGetLastError();
}

}  // namespace gs
