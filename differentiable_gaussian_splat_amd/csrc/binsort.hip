// Tile binning with a (tile, depth) key sort.
//
// Sorting the P (tile, Gaussian) pairs by the 64-bit key (tile << 32 | depth
// bits), equal keys by Gaussian index, gives each tile its Gaussians front to
// back. This file reaches exactly that order without sorting the P pairs
// (44.5M for 1M Gaussians at 1920x1080):
//   1. stable compaction of the visible Gaussians (index order kept);
//   2. LSD radix sort of those by their 32 depth bits (stable: equal depths
//      stay in index order); every tile's list is a subsequence of this order;
//   3. super-tiles of 8 x 8 tiles: each depth-sorted Gaussian emits one entry
//      per super-tile its tile rectangle meets (about 2.3 entries per Gaussian
//      at 1080p), and a stable radix pass groups the entries by super-tile,
//      keeping depth order inside each group;
//   4. one wave per piece of a super-tile's group, lane = tile of the 8 x 8
//      block: each lane tests every entry's rectangle and counts (first pass)
//      or writes the Gaussian at its own cursor (second pass). Per-piece counts,
//      their running sum per tile and a scan over tiles give the cursors, so
//      each tile receives its Gaussians in depth order with no ranking step.
// Several views of one image size are binned in one pass by stacking their
// tile grids vertically: entry i of the per-view arrays (view i / n_view)
// has its tile rectangle moved down by view x TY rows, so the tile id, and
// with it the sort key, leads with the view and no rectangle crosses a view.
// Radix passes rank stably with wave64 ballot matching against per-wave LDS
// counters and stage the block in LDS so that the output is written in
// contiguous runs. The pair counts are reduced first and copied to the host
// asynchronously, so the host's wait for them overlaps the depth sort.
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
struct StoreInPlace {
    uint32_t* p;
    __device__ void operator()(int i, u64 pos, uint32_t) const { p[i] = (uint32_t)pos; }
};
// Tile rectangle of entry i in the stacked grid of the views (nper entries
// and TYv tile rows per view; nper = 0 for a single view).
__device__ __forceinline__ void stacked_rect(int i, int nper, int TX, int TYv, float2 m, int r, int& X0, int& X1,
                                             int& Y0, int& Y1) {
    tile_rect(m.x, m.y, r, TX, TYv, X0, X1, Y0, Y1);
    const int yo = nper ? (int)((uint32_t)i / (uint32_t)nper) * TYv : 0;
    Y0 += yo;
    Y1 += yo;
}

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

// Small arrays (n <= 16K): one 1024-thread block, in chunks of SC items. A
// chunk is loaded into LDS with coalesced reads (all issued before any is
// waited on), each thread then scans a contiguous run of SC / 1024 items.
constexpr int SC = 8192;

template <class Load, class Store>
__global__ __launch_bounds__(1024) void k_scan_single(Load ld, Store st, int n, const u64* dcount, u64* total) {
    constexpr int PER = SC / 1024;
    __shared__ uint32_t s_val[SC];
    __shared__ u64 s_w[16];
    const int cnt = eff_count(n, dcount);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    u64 carry = 0;
    for (int c0 = 0; c0 < cnt; c0 += SC) {
        uint32_t v[PER];
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int i = c0 + k * 1024 + (int)threadIdx.x;
            v[k] = i < cnt ? ld(i) : 0u;
        }
#pragma unroll
        for (int k = 0; k < PER; ++k) s_val[k * 1024 + threadIdx.x] = v[k];
        __syncthreads();
        uint32_t run[PER];
        u64 sum = 0;
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            run[k] = s_val[threadIdx.x * PER + k];
            sum += run[k];
        }
        u64 x = sum;
        for (int off = 1; off < 64; off <<= 1) {
            const u64 y = __shfl_up(x, off);
            if (lane >= off) x += y;
        }
        if (lane == 63) s_w[w] = x;
        __syncthreads();
        u64 pre = 0, tot = 0;
        for (int k = 0; k < 16; ++k) {
            pre += k < w ? s_w[k] : 0ull;
            tot += s_w[k];
        }
        u64 pos = carry + pre + x - sum;
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int i = c0 + (int)threadIdx.x * PER + k;
            if (i < cnt) st(i, pos, run[k]);
            pos += run[k];
        }
        carry += tot;
        __syncthreads();  // s_val and s_w are reused by the next chunk
    }
    if (threadIdx.x == 0 && total) *total = carry;
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


// ---------------------------------------------------------------- radix sort

// One LSD pass of up to 8 bits over (key, value) pairs in memory. RB-thread
// blocks own RE consecutive elements each.
//   k_radix_hist: per-block digit counts into hist[block][digit], and the
//     digit totals added atomically into tot[RT][256] (zero on entry; block b
//     adds into row b % RT, which spreads the atomics over RT addresses);
//   k_radix_offsets (one 64-lane block per digit): the table becomes the
//     pass's output offsets, digit-major: offset[b][d] = sum over digits < d of
//     their totals + sum over blocks < b of digit d's counts. It also clears
//     the next pass's totals (spare[RT][256]), so passes alternate two buffers.
//     With up to RADIX_INLINE_BLOCKS blocks the scatter computes the same
//     offsets itself and this launch is left out;
//   k_radix_scatter: stable scatter with those offsets.
constexpr int PIECE = 256;           // super-tile entries one wave walks in the per-tile passes
constexpr int RB = 1024;             // threads per radix block (16 waves)
constexpr int RE = 4096;             // elements per radix block
constexpr int RW = RB / 64;          // waves per radix block
constexpr int RR = RE / RB;          // elements per thread
constexpr int RT = 8;                // rows of the digit-total buffers

template <class V>
struct SrcMem {
    const uint32_t* keys;
    const V* vals;
};

// Exclusive scan of v over threads 0..255 of the block (other threads pass 0
// and get 0); s_w holds 4 words.
__device__ __forceinline__ uint32_t digit_excl_scan(uint32_t v, uint32_t* s_w) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    uint32_t x = v;
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    if (lane == 63 && w < 4) s_w[w] = x;
    __syncthreads();
    uint32_t pre = 0;
    for (int i = 0; i < 4; ++i) pre += i < w ? s_w[i] : 0u;
    __syncthreads();
    return tid < 256 ? pre + x - v : 0u;
}

__global__ __launch_bounds__(RB) void k_radix_hist(const uint32_t* __restrict__ keys, int n, const u64* dcount, int shift, int bits,
                                                 uint32_t* __restrict__ hist, uint32_t* __restrict__ tot) {
    __shared__ uint32_t s_h[RW][256];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    for (int k = tid; k < RW * 256; k += RB) (&s_h[0][0])[k] = 0u;
    const int cnt = eff_count(n, dcount);
    const int p0 = blockIdx.x * RE;
    const int p1 = min(cnt, p0 + RE);
    __syncthreads();
    const uint32_t mask = (1u << bits) - 1u;
    uint32_t kk[RR];
#pragma unroll
    for (int r = 0; r < RR; ++r) {
        const int p = p0 + (w * RR + r) * 64 + lane;
        kk[r] = p < p1 ? keys[p] : 0u;
    }
#pragma unroll
    for (int r = 0; r < RR; ++r) {
        const int p = p0 + (w * RR + r) * 64 + lane;
        if (p < p1) atomicAdd(&s_h[w][(kk[r] >> shift) & mask], 1u);
    }
    __syncthreads();
    if (tid < 256) {
        uint32_t c = 0;
#pragma unroll
        for (int k = 0; k < RW; ++k) c += s_h[k][tid];
        hist[(size_t)blockIdx.x * 256 + tid] = c;
        if (c) atomicAdd(&tot[(blockIdx.x % RT) * 256 + tid], c);
    }
}

// Block d (64 lanes): digit d's base from the totals, then its running offsets
// over the blocks, each lane a contiguous run of blocks. PIECES (the one pass
// that groups super-tile entries, digit = super-tile): block d also writes
// super-tile d's entry range sr[d] = [base, base + total) and its first piece
// pfirst[d] (pieces of PIECE entries before it), and block 255 the number of
// pieces, for the per-tile passes.
template <bool PIECES>
__global__ __launch_bounds__(64) void k_radix_offsets(int nblocks, uint32_t* __restrict__ hist,
                                                    const uint32_t* __restrict__ tot, uint32_t* __restrict__ spare,
                                                    int S, uint2* __restrict__ sr, uint32_t* __restrict__ pfirst,
                                                    u64* __restrict__ npieces) {
    const int d = blockIdx.x, lane = threadIdx.x;
    // base = sum of the totals of digits below d; lane holds digits 4 lane .. 4 lane + 3
    const int j = 4 * lane;
    uint32_t t[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int r = 0; r < RT; ++r) {
        const uint4 t4 = reinterpret_cast<const uint4*>(tot + r * 256)[lane];
        t[0] += t4.x;
        t[1] += t4.y;
        t[2] += t4.z;
        t[3] += t4.w;
    }
    uint32_t below = 0, pbelow = 0, pall = 0, mine = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        below += j + i < d ? t[i] : 0u;
        if (PIECES) {
            const uint32_t pc = (t[i] + PIECE - 1) / PIECE;
            pbelow += j + i < d ? pc : 0u;
            pall += pc;
            mine += j + i == d ? t[i] : 0u;
        }
    }
    for (int off = 32; off > 0; off >>= 1) {
        below += (uint32_t)__shfl_xor((int)below, off);
        if (PIECES) {
            pbelow += (uint32_t)__shfl_xor((int)pbelow, off);
            pall += (uint32_t)__shfl_xor((int)pall, off);
            mine += (uint32_t)__shfl_xor((int)mine, off);
        }
    }
    if (PIECES && lane == 0) {
        if (d < S) {
            sr[d] = make_uint2(below, below + mine);
            pfirst[d] = pbelow;
        }
        if (d == 255) *npieces = pall;
    }
    constexpr int U = 8;
    const int per = (nblocks + 63) / 64;
    const int b0 = lane * per;
    uint32_t v[U];
    uint32_t sum = 0;
    for (int c = 0; c < per; c += U) {
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int b = b0 + c + k;
            v[k] = (c + k < per && b < nblocks) ? hist[(size_t)b * 256 + d] : 0u;
            sum += v[k];
        }
    }
    // exclusive scan of the lane sums
    uint32_t x = sum;
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = (uint32_t)__shfl_up((int)x, off);
        if (lane >= off) x += y;
    }
    uint32_t run = below + x - sum;
    for (int c = 0; c < per; c += U) {
        uint32_t w[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int b = b0 + c + k;
            w[k] = (c + k < per && b < nblocks) ? hist[(size_t)b * 256 + d] : 0u;
        }
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int b = b0 + c + k;
            if (c + k < per && b < nblocks) hist[(size_t)b * 256 + d] = run;
            run += w[k];
        }
    }
    if (lane < RT) spare[lane * 256 + d] = 0u;
}

// The super-tile table a grouping pass can write beside its offsets (see
// k_radix_offsets<true>); pfirst == nullptr: none.
struct PieceTable {
    int S = 0;
    uint2* sr = nullptr;
    uint32_t* pfirst = nullptr;
    u64* npieces = nullptr;
};

// Wave 0 of a block: digit d's first output position (the exclusive scan of
// the digit totals, summed over the RT rows of tot) into s_base[d]; with
// `table` (block 0 of a grouping pass), also the super-tile ranges, first
// pieces and piece count that k_radix_offsets<true> writes.
__device__ __forceinline__ void digit_bases(const uint32_t* __restrict__ tot, uint32_t* s_base, const PieceTable& pt,
                                            bool table) {
    const int lane = threadIdx.x & 63;
    uint32_t t[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int r = 0; r < RT; ++r) {
        const uint4 t4 = reinterpret_cast<const uint4*>(tot + r * 256)[lane];
        t[0] += t4.x;
        t[1] += t4.y;
        t[2] += t4.z;
        t[3] += t4.w;
    }
    const uint32_t sum = t[0] + t[1] + t[2] + t[3];
    uint32_t x = sum;
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = (uint32_t)__shfl_up((int)x, off);
        if (lane >= off) x += y;
    }
    uint32_t b[4];
    uint32_t run = x - sum;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        b[i] = run;
        run += t[i];
    }
    reinterpret_cast<uint4*>(s_base)[lane] = make_uint4(b[0], b[1], b[2], b[3]);
    if (table) {
        uint32_t pc[4], ps = 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            pc[i] = (t[i] + PIECE - 1) / PIECE;
            ps += pc[i];
        }
        uint32_t y = ps;
        for (int off = 1; off < 64; off <<= 1) {
            const uint32_t z = (uint32_t)__shfl_up((int)y, off);
            if (lane >= off) y += z;
        }
        uint32_t prun = y - ps;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int d = 4 * lane + i;
            if (d < pt.S) {
                pt.sr[d] = make_uint2(b[i], b[i] + t[i]);
                pt.pfirst[d] = prun;
            }
            prun += pc[i];
        }
        if (lane == 63) *pt.npieces = y;
    }
}

// Stable scatter of one digit. Wave w owns the block's elements
// [w RE/RW, (w+1) RE/RW) in rounds of 64 consecutive ones; within a round,
// lanes with equal digits are matched by ballots and ranked against the wave's
// own LDS counters (no barrier per round); after one barrier the per-digit
// wave offsets are combined, the block is reordered in LDS by (digit, rank),
// and written out so that each digit's elements form one contiguous run.
// The block's output offsets: from k_radix_offsets' table (offsets, INLINE
// false), or (INLINE) computed here from the per-block counts hist and the
// digit totals dtot: digit d's base plus its counts in the blocks before this
// one, summed by the 16 waves over rows w, w + 16, ... while the keys load;
// block 0 then also does k_radix_offsets' other work (clearing spare, the
// piece table). bstart (nullable, INLINE only): block b owns elements
// [bstart[b], bstart[b + 1]) (at most RE; the last block ends at the count)
// instead of [b RE, b RE + RE).
template <bool INLINE, class V>
__global__ __launch_bounds__(RB) void k_radix_scatter(SrcMem<V> src, int n, const u64* dcount, int shift, int bits,
                                                    const uint32_t* __restrict__ offsets,
                                                    const uint32_t* __restrict__ dtot, uint32_t* __restrict__ spare,
                                                    PieceTable pt, const u64* __restrict__ bstart,
                                                    uint32_t* __restrict__ keys_out, V* __restrict__ vals_out) {
    static_assert(sizeof(V) * RE >= 16 * RW * 64, "the waves' column sums fit in s_vals");
    __shared__ uint32_t s_keys[RE];
    __shared__ __align__(16) V s_vals[RE];  // INLINE: first the waves' column sums of hist, 256 words each
    __shared__ uint32_t s_wcnt[RW][256];  // per-wave digit counts, then each wave's first slot per digit
    __shared__ uint32_t s_dstart[256];
    __shared__ uint32_t s_gbase[256];
    __shared__ uint32_t s_base[256];
    __shared__ uint32_t s_w[4];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    if (INLINE && blockIdx.x == 0)
        for (int k = tid; k < RT * 256; k += RB) spare[k] = 0u;
    const int cnt = eff_count(n, dcount);
    int p0 = blockIdx.x * RE, p1 = min(cnt, p0 + RE);
    if (INLINE && bstart) {
        p0 = (int)bstart[blockIdx.x];
        p1 = blockIdx.x + 1 < gridDim.x ? (int)bstart[blockIdx.x + 1] : cnt;
        p1 = min(min(p1, cnt), p0 + RE);  // a consistent table keeps these
    }
    if (p0 >= p1) return;
    const uint32_t mask = (1u << bits) - 1u;
    for (int k = lane; k < 256; k += 64) s_wcnt[w][k] = 0u;
    wave_lds_sync();
    uint32_t kk[RR], rk[RR];
    V vv[RR];
    const int ebase = p0 + w * RR * 64 + lane;
#pragma unroll
    for (int r = 0; r < RR; ++r) {
        const int p = ebase + r * 64;
        kk[r] = 0u;
        vv[r] = V{};
        if (p < p1) {
            kk[r] = src.keys[p];
            vv[r] = src.vals[p];
        }
    }
    if (INLINE) {
        const uint4* h4 = reinterpret_cast<const uint4*>(offsets);
        const int b = blockIdx.x;
        constexpr int U = 16;
        uint4 acc = make_uint4(0u, 0u, 0u, 0u);
        for (int j0 = w; j0 < b; j0 += RW * U) {
            uint4 v[U];
#pragma unroll
            for (int c = 0; c < U; ++c) {
                const int j = j0 + RW * c;
                v[c] = j < b ? h4[(size_t)j * 64 + lane] : make_uint4(0u, 0u, 0u, 0u);
            }
#pragma unroll
            for (int c = 0; c < U; ++c) {
                acc.x += v[c].x;
                acc.y += v[c].y;
                acc.z += v[c].z;
                acc.w += v[c].w;
            }
        }
        reinterpret_cast<uint4*>(s_vals)[w * 64 + lane] = acc;  // read after the first barrier below
        if (w == 0) digit_bases(dtot, s_base, pt, b == 0 && pt.pfirst);
    } else if (tid < 256) {
        s_gbase[tid] = offsets[(size_t)blockIdx.x * 256 + tid];  // read after the last barrier below
    }
    const uint64_t lt = lanemask_lt();
#pragma unroll
    for (int r = 0; r < RR; ++r) {
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
    uint32_t tot = 0;
    if (tid < 256)
        for (int k = 0; k < RW; ++k) tot += s_wcnt[k][tid];
    const uint32_t ds = digit_excl_scan(tot, s_w);
    if (tid < 256) {
        s_dstart[tid] = ds;
        uint32_t run = ds;
        for (int k = 0; k < RW; ++k) {
            const uint32_t c = s_wcnt[k][tid];
            s_wcnt[k][tid] = run;
            run += c;
        }
        if (INLINE) {
            uint32_t g = s_base[tid];
#pragma unroll
            for (int k = 0; k < RW; ++k) g += reinterpret_cast<const uint32_t*>(s_vals)[k * 256 + tid];
            s_gbase[tid] = g;
        }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < RR; ++r) {
        if (ebase + r * 64 < p1) {
            const uint32_t slot = s_wcnt[w][(kk[r] >> shift) & mask] + rk[r];
            s_keys[slot] = kk[r];
            s_vals[slot] = vv[r];
        }
    }
    __syncthreads();
    const int here = p1 - p0;
    for (int sl = tid; sl < here; sl += RB) {
        const uint32_t key = s_keys[sl];
        const uint32_t d = (key >> shift) & mask;
        const uint32_t dst = s_gbase[d] + ((uint32_t)sl - s_dstart[d]);
        if (dst < (uint32_t)cnt) {  // always true for a consistent offset table
            keys_out[dst] = key;
            vals_out[dst] = s_vals[sl];
        }
    }
}

// hist: 256 words per block. rtot: two RT x 256-word total buffers; pass number
// `pass` adds into rtot[pass & 1] (zero on entry) and clears the other. Up to
// RADIX_INLINE_BLOCKS blocks the scatter computes its own offsets (the blocks
// together read nblocks^2 / 2 rows of hist); beyond, k_radix_offsets does.
constexpr int RADIX_INLINE_BLOCKS = 512;

// bstart (nullable): the histogram and digit totals are already there, for
// blocks of elements [bstart[b], bstart[b + 1]) (RADIX_INLINE_BLOCKS at most).
template <class V>
hipError_t radix_pass(SrcMem<V> src, int n, const u64* dcount, int shift, int bits, uint32_t* hist, uint32_t* rtot,
                      int pass, uint32_t* keys_out, V* vals_out, hipStream_t s, PieceTable pt = {},
                      const u64* bstart = nullptr) {
    const int nblocks = (n + RE - 1) / RE;
    if (nblocks == 0) return hipSuccess;
    uint32_t* tot = rtot + RT * 256 * (pass & 1);
    uint32_t* spare = rtot + RT * 256 * ((pass & 1) ^ 1);
    if (bstart && nblocks > RADIX_INLINE_BLOCKS) return hipErrorInvalidValue;
    if (!bstart) k_radix_hist<<<nblocks, RB, 0, s>>>(src.keys, n, dcount, shift, bits, hist, tot);
    if (nblocks <= RADIX_INLINE_BLOCKS) {
        k_radix_scatter<true, V><<<nblocks, RB, 0, s>>>(src, n, dcount, shift, bits, hist, tot, spare, pt, bstart,
                                                        keys_out, vals_out);
        return hipGetLastError();
    }
    if (pt.pfirst)
        k_radix_offsets<true><<<256, 64, 0, s>>>(nblocks, hist, tot, spare, pt.S, pt.sr, pt.pfirst, pt.npieces);
    else
        k_radix_offsets<false><<<256, 64, 0, s>>>(nblocks, hist, tot, spare, 0, nullptr, nullptr, nullptr);
    k_radix_scatter<false, V><<<nblocks, RB, 0, s>>>(src, n, dcount, shift, bits, hist, nullptr, nullptr, {},
                                                     nullptr, keys_out, vals_out);
    return hipGetLastError();
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int bits_for(int ntiles) {
    int b = 1;
    while ((1 << b) < ntiles) ++b;
    return b;
}


// ---------------------------------------------------------------- two-level tile binning

constexpr int SUPER = 8;      // a super-tile is SUPER x SUPER tiles: one wave lane per tile

__device__ __forceinline__ uint32_t super_count(int X0, int X1, int Y0, int Y1) {
    return (uint32_t)(((X1 >> 3) - (X0 >> 3) + 1) * ((Y1 >> 3) - (Y0 >> 3) + 1));
}

// P = sum of tiles_touched, P1 = number of (super-tile, Gaussian) entries and
// the number of visible Gaussians, per block of ST Gaussians (index order),
// into part[3 b .. 3 b + 2]; the compaction (k_compact_visible) totals P and
// P1 and sums the visible counts before each block itself, or, for more
// blocks than it does that for, k_pair_sum does both first. Block 0 also
// clears the radix passes' digit-total buffers.
constexpr int CT = 1024, CI = ST / CT;  // threads and items per thread of the per-Gaussian passes

__global__ __launch_bounds__(CT) void k_pair_totals(int n, const uint32_t* __restrict__ tiles,
                                                  const float2* __restrict__ means2d, const int* __restrict__ radii,
                                                  int nper, int TX, int TYv, u64* __restrict__ part,
                                                  uint32_t* __restrict__ rtot, int rtot_words) {
    __shared__ u64 s_w[3][CT / 64];
    if (blockIdx.x == 0)  // the radix passes' digit totals start at zero (the compaction adds the first)
        for (int k = threadIdx.x; k < rtot_words; k += CT) rtot[k] = 0u;
    u64 p = 0, p1 = 0, v = 0;
    const int base = blockIdx.x * ST;
    // every load issued before any is used (at a clamped index past n, not counted)
    uint32_t t[CI];
    float2 m[CI];
    int rr[CI];
#pragma unroll
    for (int j = 0; j < CI; ++j) {
        const int i = min(base + j * CT + (int)threadIdx.x, n - 1);
        t[j] = tiles[i];
        m[j] = means2d[i];
        rr[j] = radii[i];
    }
#pragma unroll
    for (int j = 0; j < CI; ++j) {
        const int i = base + j * CT + threadIdx.x;
        if (i < n && t[j]) {
            int X0, X1, Y0, Y1;
            stacked_rect(i, nper, TX, TYv, m[j], rr[j], X0, X1, Y0, Y1);
            p += t[j];
            p1 += super_count(X0, X1, Y0, Y1);
            v += 1;
        }
    }
    for (int off = 32; off > 0; off >>= 1) {
        p += __shfl_xor(p, off);
        p1 += __shfl_xor(p1, off);
        v += __shfl_xor(v, off);
    }
    if ((threadIdx.x & 63) == 0) {
        s_w[0][threadIdx.x >> 6] = p;
        s_w[1][threadIdx.x >> 6] = p1;
        s_w[2][threadIdx.x >> 6] = v;
    }
    __syncthreads();
    if (threadIdx.x < 3)
    {
        u64 t3 = 0;
        for (int k = 0; k < CT / 64; ++k) t3 += s_w[threadIdx.x][k];
        part[3 * blockIdx.x + threadIdx.x] = t3;
    }
}

// One 1024-thread block: counters[2] = P, counters[3] = P1, vis_scan[b] = the
// exclusive scan of the blocks' visible counts, counters[0] = their total;
// also clears the radix passes' digit-total buffers (rtot_words words). P and
// P1 also go straight to host[0..1]: pinned, host-coherent memory mapped into
// the device's address space, so that the host reads them after the stream's
// next event without a copy in the stream.
__global__ __launch_bounds__(1024) void k_pair_sum(int nb, const u64* __restrict__ part, u64* __restrict__ vis_scan,
                                                 u64* __restrict__ counters, uint32_t* __restrict__ rtot,
                                                 int rtot_words, u64* __restrict__ host) {
    __shared__ u64 s_w[2][16];
    __shared__ u64 s_v[16];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    for (int k = threadIdx.x; k < rtot_words; k += 1024) rtot[k] = 0u;
    u64 p = 0, p1 = 0;
    for (int i = threadIdx.x; i < nb; i += 1024) {
        p += part[3 * i];
        p1 += part[3 * i + 1];
    }
    for (int off = 32; off > 0; off >>= 1) {
        p += __shfl_xor(p, off);
        p1 += __shfl_xor(p1, off);
    }
    if (lane == 0) {
        s_w[0][w] = p;
        s_w[1][w] = p1;
    }
    // exclusive scan of the visible counts, 1024 blocks at a time
    u64 carry = 0;
    for (int b0 = 0; b0 < nb; b0 += 1024) {
        const int i = b0 + threadIdx.x;
        const u64 v = i < nb ? part[3 * i + 2] : 0ull;
        u64 x = v;
        for (int off = 1; off < 64; off <<= 1) {
            const u64 y = __shfl_up(x, off);
            if (lane >= off) x += y;
        }
        if (lane == 63) s_v[w] = x;
        __syncthreads();
        u64 pre = 0, tot = 0;
        for (int k = 0; k < 16; ++k) {
            pre += k < w ? s_v[k] : 0ull;
            tot += s_v[k];
        }
        if (i < nb) vis_scan[i] = carry + pre + x - v;
        carry += tot;
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        u64 a = 0, c = 0;
        for (int k = 0; k < 16; ++k) {
            a += s_w[0][k];
            c += s_w[1][k];
        }
        counters[0] = carry;
        counters[1] = 0ull;
        counters[2] = a;
        counters[3] = c;
        counters[4] = 0ull;
        host[0] = a;
        host[1] = c;
        __threadfence_system();
    }
}

// Stable compaction of the visible Gaussians (tiles_touched > 0), in the
// blocks of ST Gaussians that k_pair_totals counted (vis_scan[b]: visible
// ones before block b, as k_pair_sum scans them). Visible Gaussian i, the
// pos-th in index order, gets its depth bits and compact position (the depth
// sort's keys and values) and its record (index, tile rectangle X0 | X1 << 16, Y0 | Y1 << 16, depth
// bits), written here in index order so that the sorted order later gathers
// one 16-byte record each. Thread t takes Gaussians base + j CT + t, all
// loads issued up front; ranks come from one ballot per wave and row j and a
// scan of the block's 64 (row, wave) counts (index order is row, wave, lane).
//
// SELF (up to COMPACT_SELF_SUM_BLOCKS blocks, in place of k_pair_sum): vis_scan
// is k_pair_totals' table part itself; each block sums the visible counts of
// the blocks before it, writes that offset to bstart[b], and block 0 also
// does k_pair_sum's other work (the totals into counters and host).
// HIST (up to RADIX_INLINE_BLOCKS blocks): the block's visible Gaussians are
// also the first depth pass's block b (compact positions [bstart[b],
// bstart[b + 1])): their low-byte histogram goes to hist[b] and is added to
// the digit totals tot, in place of that pass's histogram kernel.
constexpr int COMPACT_SELF_SUM_BLOCKS = 4096;

template <bool SELF, bool HIST>
__global__ __launch_bounds__(CT) void k_compact_visible(int n, int nper, int TX, int TYv,
                                                      const uint32_t* __restrict__ tiles,
                                                      const float* __restrict__ depths,
                                                      const float2* __restrict__ means2d,
                                                      const int* __restrict__ radii,
                                                      const u64* __restrict__ vis_scan, uint32_t* __restrict__ keys,
                                                      uint32_t* __restrict__ idx, uint4* __restrict__ crec,
                                                      u64* __restrict__ counters, u64* __restrict__ bstart,
                                                      uint32_t* __restrict__ hist, uint32_t* __restrict__ tot,
                                                      u64* __restrict__ host) {
    static_assert(CI * (CT / 64) == 64, "one lane per (row, wave) count");
    static_assert(CT >= 256 && ST == RE, "one histogram bin per thread; a compaction block is a radix block");
    __shared__ uint32_t s_c[CI * (CT / 64)];
    __shared__ u64 s_v[CT / 64];
    __shared__ uint32_t s_h[HIST ? 256 : 1];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int base = blockIdx.x * ST;
    if (HIST && threadIdx.x < 256) s_h[threadIdx.x] = 0u;  // added to after the barrier below
    if (SELF && blockIdx.x == 0) {
        __shared__ u64 s_t[3][CT / 64];
        const int nb = gridDim.x;
        u64 p = 0, p1 = 0, v = 0;
        for (int k = threadIdx.x; k < nb; k += CT) {
            p += vis_scan[3 * k];
            p1 += vis_scan[3 * k + 1];
            v += vis_scan[3 * k + 2];
        }
        for (int off = 32; off > 0; off >>= 1) {
            p += __shfl_xor(p, off);
            p1 += __shfl_xor(p1, off);
            v += __shfl_xor(v, off);
        }
        if (lane == 0) {
            s_t[0][w] = p;
            s_t[1][w] = p1;
            s_t[2][w] = v;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            u64 a = 0, c = 0, t = 0;
            for (int k = 0; k < CT / 64; ++k) {
                a += s_t[0][k];
                c += s_t[1][k];
                t += s_t[2][k];
            }
            counters[0] = t;
            counters[1] = 0ull;
            counters[2] = a;
            counters[3] = c;
            counters[4] = 0ull;
            host[0] = a;
            host[1] = c;
            __threadfence_system();
        }
    }
    u64 vb = 0;  // SELF: visible Gaussians in the blocks before this one
    if (SELF)
        for (int k = threadIdx.x; k < (int)blockIdx.x; k += CT) vb += vis_scan[3 * k + 2];
    uint32_t t[CI], d[CI];
    float2 m[CI];
    int rr[CI];
#pragma unroll
    for (int j = 0; j < CI; ++j) {
        const int i = min(base + j * CT + (int)threadIdx.x, n - 1);  // past n: loaded, never stored
        t[j] = tiles[i];
        d[j] = __float_as_uint(depths[i]);
        m[j] = means2d[i];
        rr[j] = radii[i];
    }
    uint64_t vis[CI];
#pragma unroll
    for (int j = 0; j < CI; ++j) {
        vis[j] = __ballot(base + j * CT + (int)threadIdx.x < n && t[j] > 0u);
        if (lane == 0) s_c[j * (CT / 64) + w] = (uint32_t)__popcll(vis[j]);
    }
    if (SELF) {
        for (int off = 32; off > 0; off >>= 1) vb += __shfl_xor(vb, off);
        if (lane == 0) s_v[w] = vb;
    }
    __syncthreads();
    // lane k = (row, wave) in index order: exclusive scan of the counts
    const uint32_t c = s_c[lane];
    uint32_t x = c;
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = (uint32_t)__shfl_up((int)x, off);
        if (lane >= off) x += y;
    }
    const uint32_t excl = x - c;
    u64 boff = 0;
    if (SELF) {
#pragma unroll
        for (int k = 0; k < CT / 64; ++k) boff += s_v[k];
        if (threadIdx.x == 0) bstart[blockIdx.x] = boff;
    } else {
        boff = vis_scan[blockIdx.x];
    }
#pragma unroll
    for (int j = 0; j < CI; ++j) {
        const uint32_t first = (uint32_t)__builtin_amdgcn_readlane((int)excl, j * (CT / 64) + w);
        if ((vis[j] >> lane) & 1ull) {
            const uint32_t pos = (uint32_t)boff + first +
                                 __builtin_amdgcn_mbcnt_hi((uint32_t)(vis[j] >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)vis[j], 0u));
            const int i = base + j * CT + threadIdx.x;
            int X0, X1, Y0, Y1;
            stacked_rect(i, nper, TX, TYv, m[j], rr[j], X0, X1, Y0, Y1);
            keys[pos] = d[j];
            idx[pos] = pos;
            crec[pos] = make_uint4((uint32_t)i, (uint32_t)X0 | ((uint32_t)X1 << 16), (uint32_t)Y0 | ((uint32_t)Y1 << 16),
                                   d[j]);
            if (HIST) atomicAdd(&s_h[d[j] & 0xffu], 1u);
        }
    }
    if (HIST) {
        __syncthreads();
        if (threadIdx.x >= 256) return;
        const uint32_t c = s_h[threadIdx.x];
        hist[(size_t)blockIdx.x * 256 + threadIdx.x] = c;
        if (c) atomicAdd(&tot[(blockIdx.x % RT) * 256 + threadIdx.x], c);
    }
}

// Per depth-sorted Gaussian i (one gather of its compact record): its record
// (index, X0 | X1 << 16, Y0 | Y1 << 16, depth bits); per block of ST
// Gaussians the sum of their super-tile counts (coarse[b]), and per row of
// SB of them (row j: Gaussians base + j SB .. + SB - 1) the row's sum
// (fine[16 b + j]): the reduce step of the scan that gives each Gaussian its
// first super-tile entry. Thread t takes Gaussians base + j CT + t, so that
// row 4 j + q holds item j of waves 4 q .. 4 q + 3.
static_assert(ST == 16 * SB && CI == 4, "rows of SB Gaussians: 4 per item of a thread");

__global__ __launch_bounds__(CT) void k_sorted_records(const u64* vis_ptr, const uint32_t* __restrict__ order,
                                                     const uint4* __restrict__ crec, uint4* __restrict__ rec,
                                                     u64* __restrict__ coarse, uint32_t* __restrict__ fine) {
    __shared__ uint32_t s_f[CT / 64][CI];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int cnt = (int)*vis_ptr;
    const int base = blockIdx.x * ST;
    if (base >= cnt) {  // no Gaussian here: a zero sum, for a scan over all blocks
        if (threadIdx.x == 0) coarse[blockIdx.x] = 0ull;
        return;
    }
    // every gather issued before any is used (at a clamped index past cnt, not stored)
    uint32_t o[CI];
#pragma unroll
    for (int j = 0; j < CI; ++j) o[j] = order[min(base + j * CT + (int)threadIdx.x, cnt - 1)];
    __builtin_amdgcn_sched_barrier(0);  // all index loads in flight before the first gather waits on one
    uint4 rr[CI];
#pragma unroll
    for (int j = 0; j < CI; ++j) rr[j] = crec[o[j]];
    uint32_t v[CI];
#pragma unroll
    for (int j = 0; j < CI; ++j) {
        const int i = base + j * CT + threadIdx.x;
        v[j] = 0u;
        if (i < cnt) {
            const uint4 r = rr[j];
            rec[i] = r;
            v[j] = super_count((int)(r.y & 0xffffu), (int)(r.y >> 16), (int)(r.z & 0xffffu), (int)(r.z >> 16));
        }
    }
    // the wave's sums of its four items: two halving exchanges (masks 32, 16), four more finish
    // them, and lane l ends with item (l / 16) % 4
#pragma unroll
    for (int m = 32, k = CI / 2; m >= 16; m >>= 1, k >>= 1) {
        const bool up = (lane & m) != 0;
#pragma unroll
        for (int q = 0; q < k; ++q) {
            const uint32_t keep = up ? v[q + k] : v[q];
            const uint32_t give = up ? v[q] : v[q + k];
            v[q] = keep + (uint32_t)__shfl_xor((int)give, m);
        }
    }
#pragma unroll
    for (int m = 8; m > 0; m >>= 1) v[0] += (uint32_t)__shfl_xor((int)v[0], m);
    if ((lane & 15) == 0) s_f[w][lane >> 4] = v[0];
    __syncthreads();
    // row r = 4 j + q of SB Gaussians: item j of waves 4 q .. 4 q + 3
    if (threadIdx.x < 64) {
        uint32_t f = 0u;
        if (lane < 16) {
            const int j = lane >> 2, q = lane & 3;
#pragma unroll
            for (int k = 0; k < 4; ++k) f += s_f[4 * q + k][j];
            fine[(size_t)blockIdx.x * 16 + lane] = f;
        }
        u64 t = f;
        for (int off = 8; off > 0; off >>= 1) t += __shfl_xor(t, off);
        if (lane == 0) coarse[blockIdx.x] = t;
    }
}

// One thread per depth-sorted Gaussian, blocks of SB (block e is row e % 16
// of k_sorted_records' block e / 16). A Gaussian's first entry is the block's
// offset (the coarse sums of the scan blocks before its own, or with
// `scanned` their exclusive scan, plus the row sums before it in its own)
// plus the exclusive scan of the counts inside the block. Each wave then
// writes its Gaussians' entries 64 at a time, lane l taking the wave's entry
// e0 + l: a binary search of the wave's running counts in LDS gives the
// Gaussian and the entry's place in it, row-major over its super-tile
// rectangle, so that each store is contiguous. An entry is the super-tile id
// (the key of the grouping pass) and its payload: the Gaussian's index and
// its tile rectangle clipped to the super-tile, relative to its corner
// (cx0 | cx1 << 3 | cy0 << 6 | cy1 << 9), which is all the per-tile passes
// read of it.
// Up to EMIT_SELF_SUM_BLOCKS scan blocks every block sums the coarse sums it
// needs itself; beyond, k_scan_top scans them first.
constexpr int EMIT_SELF_SUM_BLOCKS = 512;

__global__ __launch_bounds__(SB) void k_super_emit(const u64* vis_ptr, const uint4* __restrict__ rec,
                                                 const u64* __restrict__ coarse, const uint32_t* __restrict__ fine,
                                                 int scanned, int SX, uint32_t P1, uint32_t* __restrict__ skey,
                                                 uint2* __restrict__ spay) {
    __shared__ uint32_t s_inc[SB];   // per wave: running counts of its Gaussians, inclusive
    __shared__ uint4 s_rec[SB];      // the Gaussians' records
    __shared__ uint32_t s_wid[SB];   // super-tile columns of the rectangle
    __shared__ uint32_t s_tot[SB / 64];
    __shared__ u64 s_off[SB / 64];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int cnt = (int)*vis_ptr;
    const int e = blockIdx.x;
    if (e * SB >= cnt) return;
    const int i = e * SB + tid;
    const uint4 r = rec[min(i, cnt - 1)];  // past cnt: loaded, not used
    const int q = e >> 4, row = e & 15;
    u64 off = 0;
    if (!scanned)
        for (int k = tid; k < q; k += SB) off += coarse[k];
    if (tid < row) off += fine[(size_t)q * SI + tid];
    const int sx0 = (int)(r.y & 0xffffu) >> 3, sx1 = (int)(r.y >> 16) >> 3;
    const int sy0 = (int)(r.z & 0xffffu) >> 3, sy1 = (int)(r.z >> 16) >> 3;
    const uint32_t c = i < cnt ? (uint32_t)((sx1 - sx0 + 1) * (sy1 - sy0 + 1)) : 0u;
    uint32_t x = c;
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = (uint32_t)__shfl_up((int)x, o);
        if (lane >= o) x += y;
    }
    for (int o = 32; o > 0; o >>= 1) off += __shfl_xor(off, o);
    s_inc[tid] = x;
    s_rec[tid] = r;
    s_wid[tid] = (uint32_t)(sx1 - sx0 + 1);
    if (lane == 63) s_tot[w] = x;
    if (lane == 0) s_off[w] = off;
    __syncthreads();
    u64 boff = scanned ? coarse[q] : 0ull;
    uint32_t before = 0u;
#pragma unroll
    for (int k = 0; k < SB / 64; ++k) {
        boff += s_off[k];
        before += k < w ? s_tot[k] : 0u;
    }
    const uint32_t wbase = (uint32_t)boff + before, T = s_tot[w];
    const uint32_t* inc = s_inc + w * 64;
    for (uint32_t e0 = 0; e0 < T; e0 += 64) {
        const uint32_t ent = e0 + (uint32_t)lane;
        if (ent >= T) break;
        int g = 0;  // the first of the wave's Gaussians whose running count passes ent
#pragma unroll
        for (int step = 32; step > 0; step >>= 1)
            if (inc[g + step - 1] <= ent) g += step;
        const uint32_t k = ent - (g ? inc[g - 1] : 0u);
        const uint32_t wid = s_wid[w * 64 + g];
        const uint4 gr = s_rec[w * 64 + g];
        const uint32_t dy = k / wid, dx = k - dy * wid;
        const int sx = (int)((gr.y & 0xffffu) >> 3) + (int)dx, sy = (int)((gr.z & 0xffffu) >> 3) + (int)dy;
        const int cx0 = max((int)(gr.y & 0xffffu) - SUPER * sx, 0), cx1 = min((int)(gr.y >> 16) - SUPER * sx, SUPER - 1);
        const int cy0 = max((int)(gr.z & 0xffffu) - SUPER * sy, 0), cy1 = min((int)(gr.z >> 16) - SUPER * sy, SUPER - 1);
        const uint32_t pos = wbase + ent;
        if (pos < P1) {
            skey[pos] = (uint32_t)(sy * SX + sx);
            spay[pos] = make_uint2(gr.x, (uint32_t)(cx0 | (cx1 << 3) | (cy0 << 6) | (cy1 << 9)));
        }
    }
}

// [first, last + 1) of each super-tile in the grouped entries (left at (0, 0) if empty).
__global__ __launch_bounds__(SB) void k_super_ranges(int P1, const uint32_t* __restrict__ skey, int S,
                                                   uint2* __restrict__ sr) {
    const int p = blockIdx.x * SB + threadIdx.x;
    if (p >= P1) return;
    const uint32_t s = skey[p];
    if (s >= (uint32_t)S) return;
    if (p == 0 || skey[p - 1] != s) sr[s].x = (uint32_t)p;
    if (p == P1 - 1 || skey[p + 1] != s) sr[s].y = (uint32_t)(p + 1);
}

struct LoadPieces {
    const uint2* sr;
    __device__ uint32_t operator()(int s) const {
        const uint2 r = sr[s];
        return (r.y - r.x + PIECE - 1) / PIECE;
    }
};

// The piece a wave takes: super-tile s (the last one whose first piece is at
// or before pidx) and its entry range [e0, e1).
// Up to 64 SEARCH_ROUNDS super-tiles, every lane compares a share of pfirst
// with all loads in flight at once (a ballot count per round); beyond, a
// binary search (one dependent load per step).
constexpr int SEARCH_ROUNDS = 8;

__device__ __forceinline__ void piece_of(int pidx, int S, const uint32_t* __restrict__ pfirst,
                                         const uint2* __restrict__ sr, int& s, int& e0, int& e1) {
    if (S <= 64 * SEARCH_ROUNDS) {
        const int lane = threadIdx.x & 63;
        uint32_t v[SEARCH_ROUNDS];
#pragma unroll
        for (int r = 0; r < SEARCH_ROUNDS; ++r) v[r] = lane + 64 * r < S ? pfirst[lane + 64 * r] : 0xFFFFFFFFu;
        int cnt = 0;  // super-tiles whose first piece is at or before pidx (pfirst does not decrease)
#pragma unroll
        for (int r = 0; r < SEARCH_ROUNDS; ++r) cnt += __popcll(__ballot(v[r] <= (uint32_t)pidx));
        s = cnt - 1;
    } else {
        int lo = 0, hi = S;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if ((int)pfirst[mid] <= pidx) lo = mid + 1; else hi = mid;
        }
        s = lo - 1;
    }
    const uint2 r = sr[s];
    e0 = (int)r.x + (pidx - (int)pfirst[s]) * PIECE;
    e1 = min((int)r.y, e0 + PIECE);
}

// The tiles of the super-tile that an entry's clipped rectangle (payload
// bits cx0 | cx1 << 3 | cy0 << 6 | cy1 << 9) holds: a 64-bit mask, bit
// 8 row + column; none for an invalid entry.
__device__ __forceinline__ uint64_t entry_tiles(uint32_t rc, bool valid) {
    if (!valid) return 0ull;
    const int cx0 = (int)(rc & 7u), cx1 = (int)((rc >> 3) & 7u), cy0 = (int)((rc >> 6) & 7u), cy1 = (int)((rc >> 9) & 7u);
    const uint64_t cols = (uint64_t)(((2u << cx1) - 1u) & ~((1u << cx0) - 1u));
    const uint64_t below_hi = cy1 == SUPER - 1 ? ~0ull : (1ull << (8 * (cy1 + 1))) - 1ull;
    const uint64_t rows = below_hi & ~((1ull << (8 * cy0)) - 1ull) & 0x0101010101010101ull;
    return rows * cols;
}

constexpr int PIECE_GROUPS = PIECE / 64;

// One wave per piece: for each tile l of the super-tile (lane l = 8 row +
// column), the number of the piece's entries whose rectangle holds it, to
// counts[pidx][l]. An entry's tiles inside the super-tile form a rectangle,
// so the counts are the 2D prefix sum of an 8 x 8 difference array: each
// entry adds +1 / -1 at its rectangle's corners that fall inside the super-
// tile (LDS integer atomics, exact; a corner past row or column 7 touches no
// tile), then lane l takes cell l and the running sums go along the rows and
// then the columns by lane shuffles. The piece's super-tile and entry range go
// to pinfo for the placement.
__global__ __launch_bounds__(SB) void k_tile_count(const u64* np_ptr, int S, int SX, int TX, int TY,
                                                 const uint32_t* __restrict__ pfirst, const uint2* __restrict__ sr,
                                                 const uint2* __restrict__ spay, uint32_t* __restrict__ counts,
                                                 uint4* __restrict__ pinfo) {
    __shared__ int s_diff[SB / 64][SUPER * SUPER];
    const int lane = threadIdx.x & 63;
    const int pidx = __builtin_amdgcn_readfirstlane(blockIdx.x * (SB / 64) + (int)(threadIdx.x >> 6));
    if (pidx >= (int)*np_ptr) return;  // the whole wave: no block barrier follows
    int* d = s_diff[threadIdx.x >> 6];
    d[lane] = 0;
    int s, e0, e1;
    piece_of(pidx, S, pfirst, sr, s, e0, e1);
    if (lane == 0) pinfo[pidx] = make_uint4((uint32_t)s, (uint32_t)e0, (uint32_t)e1, 0u);  // for the placement
    const int sx0 = (s % SX) * SUPER, sy0 = (s / SX) * SUPER;
    const int vw = min(SUPER, TX - sx0), vh = min(SUPER, TY - sy0);  // the super-tile's tiles inside the grid
    uint32_t rq[PIECE_GROUPS];
#pragma unroll
    for (int q = 0; q < PIECE_GROUPS; ++q) rq[q] = spay[min(e0 + 64 * q + lane, e1 - 1)].y;  // lanes past e1 repeat
    wave_lds_sync();  // the cleared array is seen before the corners are added
    // entries covering the whole super-tile (large Gaussians) share their corners: they are
    // counted with one ballot per group and added once, the others add their own corners
    int n_full = 0;
#pragma unroll
    for (int q = 0; q < PIECE_GROUPS; ++q) {
        const uint32_t rc = rq[q];
        const int cx0 = (int)(rc & 7u), cx1 = (int)((rc >> 3) & 7u), cy0 = (int)((rc >> 6) & 7u),
                  cy1 = (int)((rc >> 9) & 7u);
        const bool valid = e0 + 64 * q + lane < e1 && cx0 <= cx1 && cy0 <= cy1;
        const bool full = valid && cx0 == 0 && cy0 == 0 && cx1 == vw - 1 && cy1 == vh - 1;
        n_full += __popcll(__ballot(full));
        if (valid && !full) {
            const bool right = cx1 + 1 < SUPER, below = cy1 + 1 < SUPER;
            atomicAdd(&d[cy0 * SUPER + cx0], 1);
            if (right) atomicAdd(&d[cy0 * SUPER + cx1 + 1], -1);
            if (below) atomicAdd(&d[(cy1 + 1) * SUPER + cx0], -1);
            if (right && below) atomicAdd(&d[(cy1 + 1) * SUPER + cx1 + 1], 1);
        }
    }
    if (n_full && lane == 0) {
        atomicAdd(&d[0], n_full);
        if (vw < SUPER) atomicAdd(&d[vw], -n_full);
        if (vh < SUPER) atomicAdd(&d[vh * SUPER], -n_full);
        if (vw < SUPER && vh < SUPER) atomicAdd(&d[vh * SUPER + vw], n_full);
    }
    wave_lds_sync();
    int x = d[lane];
#pragma unroll
    for (int off = 1; off < SUPER; off <<= 1) {  // along the row: lanes 8 r .. 8 r + 7
        const int y = __shfl_up(x, off, SUPER);
        if ((lane & (SUPER - 1)) >= off) x += y;
    }
#pragma unroll
    for (int off = SUPER; off < 64; off <<= 1) {  // down the column: lanes c, c + 8, ...
        const int y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    counts[(size_t)pidx * 64 + lane] = (uint32_t)x;
}

// Placement, with the roles turned: lane = entry of a 64-entry group of the
// piece (a piece holds at most four groups), and a uniform loop over the
// super-tile's tiles that some entry of the piece holds. One block of four
// waves takes a piece: wave q loads group q's records and tile masks (bit
// 8 row + column inside the super-tile) into LDS, and after one barrier every
// wave holds all groups' masks, but only the 32-bit half with its own two rows
// of tiles (wave w: tiles 16 w .. 16 w + 15), since the per-tile loop is the
// kernel's serial part and a piece of large Gaussians visits all 64 tiles.
// For tile l, one compare per group gives the group's entries that hold it;
// their ranks (mbcnt, with the run's length so far folded in) are their slots
// in depth order (group, then lane). Without keys each group's entries store
// their Gaussians straight to those slots (one store per group, its active
// lanes on consecutive words); with keys (8-byte stores) they go through an
// LDS staging run first, which the wave then writes with every lane busy:
// there a store instruction costs the address unit about the same whatever
// its active lanes, so full ones are the cheap ones. The cursors (the tile's
// first slot plus the counts of the super-tile's earlier pieces) live one per
// lane, lane l for tile l. Slots at or past P (only with a broken invariant)
// are not written.
constexpr int PLACE_SPLIT = 4;
static_assert(SB / 64 == PLACE_SPLIT && PIECE / 64 == PLACE_SPLIT, "one wave per group and per two tile rows");

template <bool KEYS>
__global__ __launch_bounds__(SB) void k_tile_place(const u64* np_ptr, int SX, int TX, int TY,
                                                 const uint4* __restrict__ pinfo,
                                                 const uint2* __restrict__ spay, const float* __restrict__ depths,
                                                 const uint32_t* __restrict__ offs, const uint2* __restrict__ ranges,
                                                 uint32_t P, uint32_t* __restrict__ values, u64* __restrict__ keys64) {
    __shared__ uint2 s_stage[KEYS ? SB / 64 : 1][KEYS ? PIECE : 1];  // per wave: (Gaussian, depth bits) of a run
    __shared__ uint4 s_grp[PIECE_GROUPS][64];   // per group and lane: mask lo, mask hi, Gaussian, depth bits
    __shared__ uint2 s_any[PIECE_GROUPS];       // per group: OR of its masks
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    // Workgroups go to the 8 XCDs round-robin (b -> XCD b % 8); XCD x takes
    // the x-th eighth of the pieces in order, so that consecutive pieces of a
    // super-tile, whose runs meet inside cache lines, are written through the
    // same L2 and leave it as whole lines.
    const int np = (int)*np_ptr;
    const int chunk = (np + 7) >> 3;
    const int i = (int)(blockIdx.x >> 3);
    const int pidx = (int)(blockIdx.x & 7u) * chunk + i;
    if (i >= chunk || pidx >= np) return;  // the whole block: the barrier below is reached by all waves or none
    uint2* stage = s_stage[KEYS ? w : 0];
    const uint4 pi = pinfo[pidx];  // written by k_tile_count
    const int s = (int)pi.x, e0 = (int)pi.y, e1 = (int)pi.z;
    const int sx0 = (s % SX) * SUPER, sy0 = (s / SX) * SUPER;
    const int ng = (e1 - e0 + 63) / 64;
    {
        uint4 g = make_uint4(0u, 0u, 0u, 0u);
        if (w < ng) {
            const int e = e0 + 64 * w + lane;
            const uint2 pl = spay[min(e, e1 - 1)];  // lanes past e1 repeat an entry; masked out below
            const uint64_t m = entry_tiles(pl.y, e < e1);
            g = make_uint4((uint32_t)m, (uint32_t)(m >> 32), pl.x, KEYS ? __float_as_uint(depths[pl.x]) : 0u);
        }
        s_grp[w][lane] = g;
        uint32_t olo = g.x, ohi = g.y;
        for (int off = 1; off < 64; off <<= 1) {
            olo |= (uint32_t)__shfl_xor((int)olo, off);
            ohi |= (uint32_t)__shfl_xor((int)ohi, off);
        }
        if (lane == 0) s_any[w] = make_uint2(olo, ohi);
    }
    const int mtx = sx0 + (lane & 7), mty = sy0 + (lane >> 3);
    uint32_t cur = (mtx < TX && mty < TY) ? ranges[mty * TX + mtx].x + offs[(size_t)pidx * 64 + lane] : 0u;
    __syncthreads();
    // this wave's half of every group's masks: bits sh .. sh + 15 of word w / 2
    const int sh = 16 * (w & 1);
    uint32_t mw[PIECE_GROUPS], gany[PIECE_GROUPS];
    uint2 pv[PIECE_GROUPS];
    uint32_t any = 0u;
#pragma unroll
    for (int q = 0; q < PIECE_GROUPS; ++q) {
        const uint4 g = s_grp[q][lane];
        const uint2 a = s_any[q];
        mw[q] = w < 2 ? g.x : g.y;
        pv[q] = make_uint2(g.z, g.w);
        gany[q] = (uint32_t)__builtin_amdgcn_readfirstlane((int)(((w < 2 ? a.x : a.y) >> sh) & 0xffffu)) << sh;
        any |= gany[q];
    }
    uint32_t todo = any;
    while (todo) {
        const int b = __builtin_ctz(todo);
        todo &= todo - 1u;
        const uint32_t bit = 1u << b;
        const int l = 32 * (w >> 1) + b;  // the tile inside the super-tile
        if (!KEYS) {
            const uint32_t base = (uint32_t)__builtin_amdgcn_readlane((int)cur, l);
            uint32_t cnt = 0;
#pragma unroll
            for (int q = 0; q < PIECE_GROUPS; ++q) {
                if (!(gany[q] & bit)) continue;  // no entry of group q holds it (also: group q absent)
                const bool in = (mw[q] & bit) != 0u;
                const uint64_t m = __ballot(in);
                const uint32_t at =
                    base + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, cnt));
                if (in && at < P) values[at] = pv[q].x;
                cnt += (uint32_t)__popcll(m);
            }
            cur = lane == l ? base + cnt : cur;
            continue;
        }
        // pack the piece's entries holding tile l, in depth order, into the staging run
        uint32_t cnt = 0;
#pragma unroll
        for (int q = 0; q < PIECE_GROUPS; ++q) {
            if (!(gany[q] & bit)) continue;  // no entry of group q holds it (also: group q absent)
            const bool in = (mw[q] & bit) != 0u;
            const uint64_t m = __ballot(in);
            const uint32_t at = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, cnt));
            if (in) stage[at] = pv[q];
            cnt += (uint32_t)__popcll(m);
        }
        wave_lds_sync();
        const uint32_t base = (uint32_t)__builtin_amdgcn_readlane((int)cur, l);
        const u64 tkey = (u64)((sy0 + (l >> 3)) * TX + sx0 + (l & 7)) << 32;
        if ((u64)base + cnt <= (u64)P) {
            uint32_t* vdst = values + base + lane;
            u64* kdst = KEYS ? keys64 + base + lane : nullptr;
#pragma unroll
            for (int j = 0; j < PIECE / 64; ++j) {
                if ((uint32_t)(64 * j) >= cnt) break;
                if ((uint32_t)(64 * j + lane) < cnt) {
                    const uint2 e = stage[64 * j + lane];
                    vdst[64 * j] = e.x;
                    if (KEYS) kdst[64 * j] = tkey | (u64)e.y;
                }
            }
        } else {
            for (uint32_t k = (uint32_t)lane; k < cnt; k += 64) {
                const uint2 e = stage[k];
                if (base + k < P) {
                    values[base + k] = e.x;
                    if (KEYS) keys64[base + k] = tkey | (u64)e.y;
                }
            }
        }
        wave_lds_sync();  // the run is read before the next tile overwrites it
        cur = lane == l ? base + cnt : cur;
    }
}

// One block of PFX_WAVES waves per super-tile, lane = tile: running sum over
// the super-tile's pieces of the per-piece counts (in place, becoming each
// piece's offset inside the tile's run) and the tile's total. Wave w takes a
// contiguous share of the pieces: their column sums, a scan of the shares
// through LDS, then the running sums written back.
constexpr int PFX_WAVES = 16;

__global__ __launch_bounds__(64 * PFX_WAVES) void k_tile_prefix(const u64* np_ptr, int S, int SX, int TX, int TY,
                                                              const uint32_t* __restrict__ pfirst,
                                                              uint32_t* __restrict__ counts,
                                                              uint32_t* __restrict__ tile_total) {
    __shared__ uint32_t s_sum[PFX_WAVES][64];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int s = blockIdx.x;
    const int p0 = (int)pfirst[s];
    const int n = (s + 1 < S ? (int)pfirst[s + 1] : (int)*np_ptr) - p0;
    const int per = (n + PFX_WAVES - 1) / PFX_WAVES;
    const int a = p0 + min(n, w * per), b = p0 + min(n, (w + 1) * per);
    constexpr int U = 8;
    uint32_t c[U];  // the share's first U counts, kept for the second pass
    uint32_t sum = 0u;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        c[u] = a + u < b ? counts[(size_t)(a + u) * 64 + lane] : 0u;
        sum += c[u];
    }
    for (int p = a + U; p < b; p += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) sum += p + u < b ? counts[(size_t)(p + u) * 64 + lane] : 0u;
    }
    s_sum[w][lane] = sum;
    __syncthreads();
    uint32_t run = 0u, tot = 0u;
#pragma unroll
    for (int k = 0; k < PFX_WAVES; ++k) {
        const uint32_t v = s_sum[k][lane];
        run += k < w ? v : 0u;
        tot += v;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
        if (a + u < b) {
            counts[(size_t)(a + u) * 64 + lane] = run;
            run += c[u];
        }
    for (int p = a + U; p < b; p += U) {
        uint32_t d[U];
#pragma unroll
        for (int u = 0; u < U; ++u) d[u] = p + u < b ? counts[(size_t)(p + u) * 64 + lane] : 0u;
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (p + u < b) {
                counts[(size_t)(p + u) * 64 + lane] = run;
                run += d[u];
            }
    }
    const int tx = (s % SX) * SUPER + (lane & 7), ty = (s / SX) * SUPER + (lane >> 3);
    if (w == 0 && tx < TX && ty < TY) tile_total[ty * TX + tx] = tot;
}

struct Grid2 {
    int SX, SY, S;
};
Grid2 super_grid(int TX, int TY) {
    Grid2 g;
    g.SX = (TX + SUPER - 1) / SUPER;
    g.SY = (TY + SUPER - 1) / SUPER;
    g.S = g.SX * g.SY;
    return g;
}

// Counters (u64): [0] visible, [1] zero, [2] P, [3] P1, [4] pieces.
constexpr int NCOUNTERS = 8;

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
    const size_t nn = (size_t)(n > 0 ? n : 1), cap = (size_t)(capacity > 0 ? capacity : 1);
    const size_t ntiles = (size_t)TX * TY;
    const Grid2 G = super_grid(TX, TY);
    const size_t S = (size_t)G.S;
    const size_t max_pieces = (cap + PIECE - 1) / PIECE + S;
    L.dkeys[0] = take(4 * nn);
    L.dkeys[1] = take(4 * nn);
    L.didx[0] = take(4 * nn);
    L.didx[1] = take(4 * nn);
    L.rec = take(16 * nn);
    L.crec = take(16 * nn);
    L.skey[0] = take(4 * cap);  // super entries: at most one per pair
    L.skey[1] = take(4 * cap);
    L.sval[0] = take(8 * cap);  // payloads: Gaussian, clipped rectangle
    L.sval[1] = take(8 * cap);
    L.sranges = take(8 * S);
    L.pfirst = take(4 * (S + 1));
    L.counts = take(4 * 64 * max_pieces);
    L.pinfo = take(16 * max_pieces);
    L.tile_total = take(4 * ntiles);
    size_t max_elems = nn > cap ? nn : cap;
    const size_t hist_entries = 256 * ((max_elems + RE - 1) / RE);
    size_t max_scan = hist_entries;
    if (nn > max_scan) max_scan = nn;
    if (ntiles > max_scan) max_scan = ntiles;
    if (S > max_scan) max_scan = S;
    L.partials = take(8 * ((max_scan + ST - 1) / ST + 1));
    L.pair_part = take(8 * 3 * ((nn + ST - 1) / ST));
    L.fine = take(4 * SI * ((nn + ST - 1) / ST));
    L.hist = take(4 * hist_entries);
    L.counters = take(8 * NCOUNTERS + 4 * 2 * RT * 256);  // counters, then the radix passes' two digit-total buffers
    L.total = off;
    return L;
}

hipError_t launch_bin_count(int n, int nper, int TX, int TYv, const float* means2d, const int* radii,
                            const float* depths, const uint32_t* tiles_touched, char* ws, const BinLayout& L,
                            unsigned long long* mapped_counts, hipEvent_t ev, hipStream_t s) {
    u64* counters = reinterpret_cast<u64*>(ws + L.counters);
    u64* partials = reinterpret_cast<u64*>(ws + L.partials);
    const float2* m2 = reinterpret_cast<const float2*>(means2d);
    uint32_t* rtot = reinterpret_cast<uint32_t*>(ws + L.counters) + 2 * NCOUNTERS;
    const int rtot_words = 2 * RT * 256;
    u64* host = reinterpret_cast<u64*>(mapped_counts);
    hipError_t e = hipSuccess;
    if (n == 0) {  // no blocks: the totals are zero
        k_pair_sum<<<1, 1024, 0, s>>>(0, nullptr, partials, counters, rtot, rtot_words, host);
        e = hipGetLastError();
        if (e == hipSuccess) e = hipEventRecord(ev, s);
        return e;
    }
    // the pair counts first, on their way to the host while the rest runs; the
    // same pass counts the visible Gaussians per block for the compaction, and
    // clears both radix total buffers (the depth sort's four passes leave
    // buffer 0 clear again for the super-tile pass of launch_bin_emit). Up to
    // COMPACT_SELF_SUM_BLOCKS blocks the compaction does k_pair_sum's work.
    const int nb = (n + ST - 1) / ST;
    const bool self_sum = nb <= COMPACT_SELF_SUM_BLOCKS;
    u64* part = reinterpret_cast<u64*>(ws + L.pair_part);
    k_pair_totals<<<nb, CT, 0, s>>>(n, tiles_touched, m2, radii, nper, TX, TYv, part, rtot, rtot_words);
    if (!self_sum) {
        k_pair_sum<<<1, 1024, 0, s>>>(nb, part, partials, counters, rtot, rtot_words, host);
        e = hipGetLastError();
        if (e == hipSuccess) e = hipEventRecord(ev, s);
        if (e != hipSuccess) return e;
    }
    uint32_t* dk[2] = {reinterpret_cast<uint32_t*>(ws + L.dkeys[0]), reinterpret_cast<uint32_t*>(ws + L.dkeys[1])};
    uint32_t* di[2] = {reinterpret_cast<uint32_t*>(ws + L.didx[0]), reinterpret_cast<uint32_t*>(ws + L.didx[1])};
    // 1. visible compaction (index order kept): depth bits, compact positions, records
    uint4* crec = reinterpret_cast<uint4*>(ws + L.crec);
    uint32_t* hist = reinterpret_cast<uint32_t*>(ws + L.hist);
    // up to RADIX_INLINE_BLOCKS blocks the compaction also histograms the first
    // depth pass, whose blocks are then the compaction's (starts in partials)
    const bool first_hist = nb <= RADIX_INLINE_BLOCKS;
    if (self_sum && first_hist)
        k_compact_visible<true, true><<<nb, CT, 0, s>>>(n, nper, TX, TYv, tiles_touched, depths, m2, radii, part,
                                                        dk[0], di[0], crec, counters, partials, hist, rtot, host);
    else if (self_sum)
        k_compact_visible<true, false><<<nb, CT, 0, s>>>(n, nper, TX, TYv, tiles_touched, depths, m2, radii, part,
                                                         dk[0], di[0], crec, counters, partials, nullptr, nullptr,
                                                         host);
    else
        k_compact_visible<false, false><<<nb, CT, 0, s>>>(n, nper, TX, TYv, tiles_touched, depths, m2, radii,
                                                          partials, dk[0], di[0], crec, nullptr, nullptr, nullptr,
                                                          nullptr, nullptr);
    e = hipGetLastError();
    if (e == hipSuccess && self_sum) e = hipEventRecord(ev, s);
    if (e != hipSuccess) return e;
    // 2. stable sort by the 32 depth bits, 4 passes of 8: the result returns to buffer 0
    for (int pass = 0; pass < 4; ++pass) {
        int c = pass & 1;
        e = radix_pass(SrcMem<uint32_t>{dk[c], di[c]}, n, &counters[0], 8 * pass, 8, hist, rtot, pass, dk[c ^ 1],
                       di[c ^ 1], s, PieceTable{}, pass == 0 && self_sum && first_hist ? partials : nullptr);
        if (e != hipSuccess) return e;
    }
    // 3. per depth-sorted Gaussian its record, and per block of them the sum of
    //    their super-tile counts (scanned here only for more blocks than
    //    k_super_emit sums itself)
    uint4* rec = reinterpret_cast<uint4*>(ws + L.rec);
    uint32_t* fine = reinterpret_cast<uint32_t*>(ws + L.fine);
    k_sorted_records<<<nb, CT, 0, s>>>(&counters[0], di[0], crec, rec, partials, fine);
    if (nb > EMIT_SELF_SUM_BLOCKS) k_scan_top<<<1, 1024, 0, s>>>(partials, nb, nullptr);
    return hipGetLastError();
}

hipError_t launch_bin_emit(int n, int P, int P1, int TX, int TY, const float* depths, char* ws, const BinLayout& L,
                           uint64_t* keys, uint32_t* values, uint32_t* ranges, hipStream_t s) {
    const int ntiles = TX * TY;
    if (P == 0 || n == 0 || P1 == 0) return fill(ranges, (size_t)2 * ntiles, 0u, s);
    u64* counters = reinterpret_cast<u64*>(ws + L.counters);
    u64* partials = reinterpret_cast<u64*>(ws + L.partials);
    uint32_t* hist = reinterpret_cast<uint32_t*>(ws + L.hist);
    uint32_t* rtot = reinterpret_cast<uint32_t*>(ws + L.counters) + 2 * NCOUNTERS;
    const uint4* rec = reinterpret_cast<const uint4*>(ws + L.rec);
    uint32_t* sk[2] = {reinterpret_cast<uint32_t*>(ws + L.skey[0]), reinterpret_cast<uint32_t*>(ws + L.skey[1])};
    uint2* sv[2] = {reinterpret_cast<uint2*>(ws + L.sval[0]), reinterpret_cast<uint2*>(ws + L.sval[1])};
    uint2* sr = reinterpret_cast<uint2*>(ws + L.sranges);
    uint32_t* pfirst = reinterpret_cast<uint32_t*>(ws + L.pfirst);
    uint32_t* counts = reinterpret_cast<uint32_t*>(ws + L.counts);
    uint32_t* tile_total = reinterpret_cast<uint32_t*>(ws + L.tile_total);
    uint4* pinfo = reinterpret_cast<uint4*>(ws + L.pinfo);
    const Grid2 G = super_grid(TX, TY);

    // 3. super-tile entries in depth order, then grouped by super-tile (stable)
    const int nb = (n + ST - 1) / ST;
    const uint32_t* fine = reinterpret_cast<const uint32_t*>(ws + L.fine);
    k_super_emit<<<(n + SB - 1) / SB, SB, 0, s>>>(&counters[0], rec, partials, fine, nb > EMIT_SELF_SUM_BLOCKS, G.SX,
                                                  (uint32_t)P1, sk[0], sv[0]);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int sbits = bits_for(G.S);
    const int passes = (sbits + 7) / 8;
    const int bpp = (sbits + passes - 1) / passes;
    int cur = 0;
    // with one pass (up to 256 super-tiles) its digit totals are the super-tiles' entry counts: the pass
    // writes their ranges and first pieces itself
    const PieceTable pt{G.S, sr, pfirst, &counters[4]};
    for (int pass = 0; pass < passes; ++pass) {
        const int shift = pass * bpp;
        const int bits = min(bpp, sbits - shift);
        e = radix_pass(SrcMem<uint2>{sk[cur], sv[cur]}, P1, nullptr, shift, bits, hist, rtot, pass, sk[cur ^ 1], sv[cur ^ 1], s,
                       passes == 1 ? pt : PieceTable{});
        if (e != hipSuccess) return e;
        cur ^= 1;
    }
    if (passes > 1) {
        e = fill(reinterpret_cast<uint32_t*>(sr), (size_t)2 * G.S, 0u, s);
        if (e != hipSuccess) return e;
        k_super_ranges<<<(P1 + SB - 1) / SB, SB, 0, s>>>(P1, sk[cur], G.S, sr);
        // pieces of PIECE entries, per super-tile
        e = scan(LoadPieces{sr}, StoreInPlace{pfirst}, G.S, nullptr, partials, &counters[4], s);
        if (e != hipSuccess) return e;
    }
    // 4. per-tile counts per piece, their running sums and tile totals, tile ranges, placement
    const int max_pieces = (P1 + PIECE - 1) / PIECE + G.S;
    const int wpb = SB / 64;
    k_tile_count<<<(max_pieces + wpb - 1) / wpb, SB, 0, s>>>(&counters[4], G.S, G.SX, TX, TY, pfirst, sr, sv[cur],
                                                             counts, pinfo);
    k_tile_prefix<<<G.S, 64 * PFX_WAVES, 0, s>>>(&counters[4], G.S, G.SX, TX, TY, pfirst, counts, tile_total);
    e = scan(LoadPlain{tile_total}, StoreRanges{reinterpret_cast<uint2*>(ranges)}, ntiles, nullptr, partials, nullptr,
             s);
    if (e != hipSuccess) return e;
    if (keys)
        k_tile_place<true><<<8 * ((max_pieces + 7) / 8), SB, 0, s>>>(
            &counters[4], G.SX, TX, TY, pinfo, sv[cur], depths, counts,
            reinterpret_cast<const uint2*>(ranges), (uint32_t)P, values, reinterpret_cast<u64*>(keys));
    else
        k_tile_place<false><<<8 * ((max_pieces + 7) / 8), SB, 0, s>>>(
            &counters[4], G.SX, TX, TY, pinfo, sv[cur], nullptr, counts,
            reinterpret_cast<const uint2*>(ranges), (uint32_t)P, values, nullptr);
    return hipGetLastError();
}

}  // namespace gs
