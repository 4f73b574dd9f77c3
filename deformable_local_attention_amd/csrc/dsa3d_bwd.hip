// dsa3d_bwd.hip -- 3D-DSA backward for gfx950, without atomics on the gradients.
//
// The gradient of one sample p of query x (head eta) reaches the query side
// (dq, doffsets) and the eight key/value rows at the corners of its trilinear
// cell. Pushing those corner contributions with atomics costs 16*head_dim
// atomic adds per sample; instead the backward pulls them per key:
//
//  1. count kernel: the base cell floor(pos) of every sample (geometry only),
//     counted per tile of tokens in an LDS histogram whose non-zero cells are
//     then added to the buckets' 32-bit counts;
//  2. an exclusive scan turns the counts into bucket starts, which also
//     replace the counts as the buckets' fill cursors;
//  3. query kernel (one task = one (query, head), as in the forward):
//     recompute the logits, a_p = exp(s_p - lse), da_p = sum_c w_c <dO, V[c]>,
//     ds_p = a_p (da_p - <dO, o>); write dq = scale sum_p ds_p sum_c w_c K[c]
//     and doffsets; and write per sample a 32-byte record (scale*ds_p, a_p,
//     the fraction f, the query token, the sample number) straight into a free
//     slot of its bucket (one more atomic on the cursor);
//  4. deterministic mode only: sort every bucket by sample number, so that the
//     summation order below does not depend on the order the slots were taken
//     (a bucket holds P records on average; one wave ranks a bucket of up to
//     128 in registers);
//  5. key kernel (one task = a 2 x 2 group of keys of one head, in t and w):
//     the samples whose cell has key y as corner c are exactly those with
//     base cell y - c, so a key streams the records of the 8 buckets y - c
//     and accumulates
//        dK[y] += w_c * scale * ds_p * q_x,   dV[y] += w_c * a_p * dO_x
//     in float32 registers, then writes its rows once; the four keys of a
//     group share buckets and read each shared record and row once.
// Base cells run over the grid extended by one cell on the low side of each
// axis (a cell with base -1 still has its upper corner at 0), per (batch,
// head). A pass covers a range of heads whose index fits in the workspace;
// sample and cell numbers are 32-bit within a pass.
#include "dsa3d_attn_common.h"
#include "dsa3d_internal.h"

#include <type_traits>

namespace dsa3d {

constexpr int kScanThreads = 256;
constexpr int kScanItems = 16;
constexpr uint32_t kScanChunk = kScanThreads * kScanItems;
constexpr uint32_t kWaveSortMax = 512;  // buckets up to this size: one wave, in LDS
constexpr int kSortBucketsPerBlock = 64;
constexpr uint32_t kNoSlot = 0xffffffffu;  // a sample with no record

// Per-sample record, written by the query kernel into its bucket and read by
// the key kernel.
struct __attribute__((aligned(16))) SampleRec {
    float ck;          // scale * ds_p
    float cv;          // a_p
    float ft, fh, fw;
    uint32_t sid;      // sample number within the pass: task * P + p
    uint32_t row_lo;   // byte offset of the query's row, token * heads * head_dim * elem_size
    uint32_t row_hi;   // (split in two words)
};

struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* off;
    const void* o;
    const void* dout;
    const float* lse;
    void* dq;
    void* doff;
    void* dk;
    void* dv;
    uint32_t* cnt;    // [ncell] bucket counts, then fill cursors (the next free record of each bucket)
    uint32_t* start;  // [ncell + 1] bucket starts
    SampleRec* rec;   // [nsamp] records, bucket by bucket
    uint32_t nsamp;   // records in this pass
    TaskGrid g;
    BlockOrder ord;
    int32_t P;
    float scale;
    Window win;
};

__device__ __forceinline__ uint32_t cell_index(const TaskGrid& g, int64_t bh, int32_t t0, int32_t h0, int32_t w0) {
    return (uint32_t)((((bh * (g.T + 1) + (t0 + 1)) * (g.H + 1) + (h0 + 1)) * (int64_t)(g.W + 1)) + (w0 + 1));
}

// ---------------------------------------------------------------------------
// 1. count kernel: one thread per sample, in sample-number order
// ---------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(256) dsa3d_bwd_count_kernel(BwdArgs a) {
    const uint64_t nsamp = (uint64_t)a.g.ntasks * a.P;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nsamp; i += (uint64_t)gridDim.x * blockDim.x) {
        const int64_t task = (int64_t)(i / (uint32_t)a.P);
        const int32_t p = (int32_t)(i - (uint64_t)task * a.P);
        int32_t b, eta, t, h, w;
        int64_t tok;
        task_coords(a.g, task, b, eta, t, h, w, tok);
        float dt, dh, dw;
        load_offsets<T>(reinterpret_cast<const T*>(a.off) + ((tok * a.g.heads + eta) * (int64_t)a.P + p) * 3, dt, dh,
                        dw);
        int32_t t0, h0, w0;
        float ft, fh, fw;
        if (!sample_geometry(a.win, t, h, w, p, dt, dh, dw, t0, h0, w0, ft, fh, fw)) continue;
        if (t0 < -1 || t0 >= a.g.T || h0 < -1 || h0 >= a.g.H || w0 < -1 || w0 >= a.g.W) continue;
        const int64_t bh = (int64_t)b * a.g.nheads + (eta - a.g.head0);
        atomicAdd(a.cnt + cell_index(a.g, bh, t0, h0, w0), 1u);
    }
}

// The same counts, tile by tile: a block takes 4 frames x 8 rows x 16 tokens
// of one (batch, head) and counts its samples' cells in an LDS histogram over
// the tile's cells widened by the window's reach plus a margin, then adds the
// histogram's non-zero entries to the global counts (one atomic per cell
// instead of one per sample); a sample whose cell lies outside the histogram
// counts in global memory directly. Counts are integers, so the result does
// not depend on the order.
constexpr int kCtT = 4, kCtH = 8, kCtW = 16;
constexpr int kCountLdsCells = 12288;  // 48 KiB

struct CountTile {
    int32_t mt, mh, mw;     // reach of a sample beyond its token, in cells, per axis
    int32_t RT, RH, RW;     // histogram extent: tile + 2*reach + 1 (cells start one below a token)
    int32_t ntt, nth, ntw;  // tiles per axis
};

template <typename T>
__global__ void __launch_bounds__(256) dsa3d_bwd_count_tiled_kernel(BwdArgs a, CountTile ct) {
    __shared__ uint32_t hist[kCountLdsCells];
    const int ncell = ct.RT * ct.RH * ct.RW;
    for (int i = threadIdx.x; i < ncell; i += 256) hist[i] = 0u;
    __syncthreads();
    const int64_t per_bh = (int64_t)ct.ntt * ct.nth * ct.ntw;
    const int64_t bh = blockIdx.x / per_bh;
    const int32_t r = (int32_t)(blockIdx.x - bh * per_bh);
    const int32_t it = r / (ct.nth * ct.ntw), ih = (r / ct.ntw) % ct.nth, iw = r % ct.ntw;
    const int32_t tt0 = it * kCtT, th0 = ih * kCtH, tw0 = iw * kCtW;
    const int32_t ot = tt0 - ct.mt - 1, oh = th0 - ct.mh - 1, ow = tw0 - ct.mw - 1;  // histogram origin
    const int32_t b = (int32_t)(bh / a.g.nheads);
    const int32_t eta = a.g.head0 + (int32_t)(bh - (int64_t)b * a.g.nheads);
    const uint32_t tok_b = (uint32_t)b * (uint32_t)a.g.T * (uint32_t)a.g.H * (uint32_t)a.g.W;
    const int nsamp = kCtT * kCtH * kCtW * a.P;
    for (int i = threadIdx.x; i < nsamp; i += 256) {
        const int lt = i / a.P, p = i - lt * a.P;
        const int32_t t = tt0 + lt / (kCtH * kCtW), h = th0 + (lt / kCtW) % kCtH, w = tw0 + lt % kCtW;
        if (t >= a.g.T || h >= a.g.H || w >= a.g.W) continue;
        const int64_t tok = (int64_t)tok_b + ((int64_t)t * a.g.H + h) * a.g.W + w;
        float dt, dh, dw;
        load_offsets<T>(reinterpret_cast<const T*>(a.off) + ((tok * a.g.heads + eta) * (int64_t)a.P + p) * 3, dt, dh,
                        dw);
        int32_t t0, h0, w0;
        float ft, fh, fw;
        if (!sample_geometry(a.win, t, h, w, p, dt, dh, dw, t0, h0, w0, ft, fh, fw)) continue;
        if (t0 < -1 || t0 >= a.g.T || h0 < -1 || h0 >= a.g.H || w0 < -1 || w0 >= a.g.W) continue;
        const uint32_t lt0 = (uint32_t)(t0 - ot), lh0 = (uint32_t)(h0 - oh), lw0 = (uint32_t)(w0 - ow);
        if (lt0 < (uint32_t)ct.RT && lh0 < (uint32_t)ct.RH && lw0 < (uint32_t)ct.RW)
            atomicAdd(&hist[(lt0 * ct.RH + lh0) * ct.RW + lw0], 1u);
        else
            atomicAdd(a.cnt + cell_index(a.g, bh, t0, h0, w0), 1u);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < ncell; i += 256) {
        const uint32_t c = hist[i];
        if (c == 0u) continue;  // only cells that samples counted, all inside the grid's cell range
        const int32_t lw0 = i % ct.RW, lh0 = (i / ct.RW) % ct.RH, lt0 = i / (ct.RW * ct.RH);
        atomicAdd(a.cnt + cell_index(a.g, bh, ot + lt0, oh + lh0, ow + lw0), c);
    }
}

// ---------------------------------------------------------------------------
// 2. exclusive scan of the bucket counts: start[i] = sum_{j<i} cnt[j],
//    start[n] = total. Three kernels: chunk sums, a one-block scan of the chunk
//    sums, and the chunk-local scans.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t x, uint32_t* lds, uint32_t& total) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
    uint32_t incl = x;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
    }
    if (lane == 63) lds[wid] = incl;
    __syncthreads();
    if (wid == 0) {
        const uint32_t v = lane < nw ? lds[lane] : 0u;
        uint32_t inc = v;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const uint32_t y = __shfl_up(inc, o, 64);
            if (lane >= o) inc += y;
        }
        if (lane < nw) lds[lane] = inc - v;
        if (lane == nw - 1) lds[nw] = inc;
    }
    __syncthreads();
    const uint32_t excl = incl - x + lds[wid];
    total = lds[nw];
    __syncthreads();
    return excl;
}

__global__ void __launch_bounds__(kScanThreads) dsa3d_scan_sums_kernel(const uint32_t* cnt, uint32_t n, uint32_t* bsum) {
    __shared__ uint32_t lds[kScanThreads / 64 + 1];
    const uint64_t i0 = (uint64_t)blockIdx.x * kScanChunk + (uint64_t)threadIdx.x * kScanItems;
    uint32_t s = 0;
#pragma unroll
    for (int j = 0; j < kScanItems; ++j)
        if (i0 + j < n) s += cnt[i0 + j];
    uint32_t total;
    (void)block_exclusive_scan(s, lds, total);
    if (threadIdx.x == 0) bsum[blockIdx.x] = total;
}

__global__ void __launch_bounds__(1024) dsa3d_scan_top_kernel(uint32_t* bsum, uint32_t nb, uint32_t* start, uint32_t n) {
    __shared__ uint32_t lds[1024 / 64 + 1];
    uint32_t carry = 0;
    for (uint32_t base = 0; base < nb; base += 1024) {
        const uint32_t i = base + threadIdx.x;
        const uint32_t x = i < nb ? bsum[i] : 0u;
        uint32_t total;
        const uint32_t e = block_exclusive_scan(x, lds, total);
        if (i < nb) bsum[i] = carry + e;
        carry += total;
    }
    if (threadIdx.x == 0) start[n] = carry;
}

// The chunk-local scans write each bucket's start twice: into `start`, and
// over its count, which from then on is the bucket's fill cursor.
__global__ void __launch_bounds__(kScanThreads) dsa3d_scan_apply_kernel(uint32_t* cnt, uint32_t n,
                                                                        const uint32_t* bsum, uint32_t* start) {
    __shared__ uint32_t lds[kScanThreads / 64 + 1];
    const uint64_t i0 = (uint64_t)blockIdx.x * kScanChunk + (uint64_t)threadIdx.x * kScanItems;
    uint32_t x[kScanItems];
    uint32_t s = 0;
#pragma unroll
    for (int j = 0; j < kScanItems; ++j) {
        x[j] = i0 + j < n ? cnt[i0 + j] : 0u;
        s += x[j];
    }
    uint32_t total;
    uint32_t run = block_exclusive_scan(s, lds, total) + bsum[blockIdx.x];
#pragma unroll
    for (int j = 0; j < kScanItems; ++j) {
        if (i0 + j < n) { start[i0 + j] = run; cnt[i0 + j] = run; }
        run += x[j];
    }
}

// ---------------------------------------------------------------------------
// 3. query kernel
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ void __launch_bounds__(256) dsa3d_bwd_query_kernel(BwdArgs a) {
    constexpr int L = D / 8;
    const int g = threadIdx.x / L;
    const int li = threadIdx.x % L;
    int64_t bh;
    int32_t t, h, wb;
    block_coords(a.g, a.ord, logical_block(blockIdx.x, gridDim.x, a.ord.chunk), bh, t, h, wb);
    const int32_t w = wb + g;
    if (w >= a.g.W) return;  // no block-wide barrier below
    const int32_t b = (int32_t)(bh / a.g.nheads);
    const int32_t eta = a.g.head0 + (int32_t)(bh - (int64_t)b * a.g.nheads);
    const uint32_t tok_b = (uint32_t)b * (uint32_t)a.g.T * (uint32_t)a.g.H * (uint32_t)a.g.W;
    const int64_t tok = (int64_t)tok_b + ((int64_t)t * a.g.H + h) * a.g.W + w;
    const int64_t task = ((bh * a.g.T + t) * a.g.H + h) * (int64_t)a.g.W + w;
    const int64_t C = (int64_t)a.g.heads * D;
    const int64_t row_off = (int64_t)eta * D + li * 8;
    const CornerStrides cs = corner_strides(a.g, C * (int64_t)sizeof(T));
    const char* Kb = reinterpret_cast<const char*>(reinterpret_cast<const T*>(a.k) + row_off);
    const char* Vb = reinterpret_cast<const char*>(reinterpret_cast<const T*>(a.v) + row_off);
    const char* zero = reinterpret_cast<const char*>(g_zero_row);
    const int64_t offrow = (tok * a.g.heads + eta) * (int64_t)a.P * 3;
    const T* offq = reinterpret_cast<const T*>(a.off) + offrow;
    T* doffq = reinterpret_cast<T*>(a.doff) + offrow;
    const uint32_t sid0 = (uint32_t)(task * a.P);
    const uint64_t qrow_bytes = (uint64_t)tok * (uint64_t)cs.row_bytes;

    Frag8<T> qf, gf, of;
    qf.load(reinterpret_cast<const T*>(a.q) + tok * C + row_off);
    gf.load(reinterpret_cast<const T*>(a.dout) + tok * C + row_off);
    of.load(reinterpret_cast<const T*>(a.o) + tok * C + row_off);
    const float Dsum = group_sum<L>(gf.dot(of, 0.0f));
    const float lse = a.lse[tok * a.g.heads + eta];

    // Chunks of L samples: each lane computes one sample's cell and takes the
    // next record of the cell's bucket from its cursor (so a chunk's atomics
    // issue together), the
    // group then works through the chunk sample by sample while the slots
    // return, and finally each lane writes its own sample's doffsets and
    // record.
    __shared__ SampleGeo s_geo[256];
    __shared__ float4 s_out[256];   // scale*ds_p, a_p, doff_t, doff_h
    __shared__ float s_outw[256];   // doff_w
    __shared__ uint4 s_rec[256][2]; // the chunk's records, staged for paired stores
    __shared__ uint32_t s_slot[256]; // their slots (kNoSlot: none)
    SampleGeo* geo = s_geo + (threadIdx.x - li);
    float4* out = s_out + (threadIdx.x - li);
    float* outw = s_outw + (threadIdx.x - li);

    float dq[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int p0 = 0; p0 < a.P; p0 += L) {
        const int n = min(L, a.P - p0);
        wave_lds_sync();  // the previous chunk has been read and flushed
        bool has_rec = false;
        uint32_t slot = 0u;  // the record taken from the bucket's cursor
        if (li < n) {
            SampleGeo sg;
            int32_t t0, h0, w0;
            sample_geo<T>(a.g, a.win, tok_b, t, h, w, p0 + li, offq + (p0 + li) * 3, sg, t0, h0, w0);
            if ((sg.valid & 0xffu) != 0u) {
                const uint32_t cell = cell_index(a.g, bh, t0, h0, w0);
                slot = atomicAdd(a.cnt + cell, 1u);
                has_rec = true;
            }
            geo[li] = sg;
        }
        wave_lds_sync();
        for (int j = 0; j < n; ++j) {
            const SampleGeo& sg = geo[j];
            const uint32_t valid = sg.valid;
            CornerAddr ca;
            corner_addresses(sg.tok0, valid, Kb, Vb, cs, zero, __all((valid >> 8) & 1u), ca);
            Frag8<T> kf[8], vf[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                kf[i].load(reinterpret_cast<const T*>(ca.a[i]));
                vf[i].load(reinterpret_cast<const T*>(ca.b[i]));
            }
            float qk[8], dv[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                qk[i] = kf[i].dot(qf, 0.0f);
                dv[i] = vf[i].dot(gf, 0.0f);
            }
            // The logit, dL/da and the derivatives of both along t, h, w, in
            // factored form over the cell's axes (w, then h, then t). The raw
            // factors (1-f, f) serve every corner: a corner outside the grid
            // read a zero row, so its dot products are exactly 0.
            const float ft = sg.ft, fh = sg.fh, fw = sg.fw;
            const float aw0 = 1.0f - fw, ah0 = 1.0f - fh, at0 = 1.0f - ft;
            float r[8];
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                const float* X = x == 0 ? qk : dv;
                float A[4], dW[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {  // k = ct*2 + ch
                    A[k] = fmaf(fw, X[2 * k + 1], aw0 * X[2 * k]);
                    dW[k] = X[2 * k + 1] - X[2 * k];
                }
                const float B0 = fmaf(fh, A[1], ah0 * A[0]), B1 = fmaf(fh, A[3], ah0 * A[2]);
                r[x] = fmaf(ft, B1, at0 * B0);                                        // value
                r[2 + 3 * x] = B1 - B0;                                                // d/dt
                r[3 + 3 * x] = fmaf(ft, A[3] - A[2], at0 * (A[1] - A[0]));            // d/dh
                r[4 + 3 * x] = fmaf(ft, fmaf(fh, dW[3], ah0 * dW[2]), at0 * fmaf(fh, dW[1], ah0 * dW[0]));  // d/dw
            }
            // r = {value(qk), value(dv), d/dt(qk), d/dh(qk), d/dw(qk), d/dt(dv), d/dh(dv), d/dw(dv)}
#pragma unroll
            for (int k = 0; k < 8; ++k) r[k] = group_sum<L>(r[k]);
            const float s = a.scale * r[0];
            const float ap = __expf(s - lse);
            const float ds = ap * (r[1] - Dsum);
            const float ck = a.scale * ds;
#pragma unroll
            for (int i = 0; i < 8; ++i) kf[i].axpy(ck * sg.w[i], dq);
            if (li == 0) {
                out[j] = make_float4(ck, ap, fmaf(ck, r[2], ap * r[5]), fmaf(ck, r[3], ap * r[6]));
                outw[j] = fmaf(ck, r[4], ap * r[7]);
            }
        }
        wave_lds_sync();
        uint32_t my_slot = kNoSlot;
        if (li < n) {
            const int p = p0 + li;
            const float4 ov = out[li];
            store_scalar<T>(doffq + p * 3 + 0, ov.z);
            store_scalar<T>(doffq + p * 3 + 1, ov.w);
            store_scalar<T>(doffq + p * 3 + 2, outw[li]);
            const SampleGeo& sg = geo[li];
            // the count kernel filed exactly these samples in these cells, so
            // the slot lies in the sample's bucket; the bound only keeps a
            // write inside the records
            if (has_rec && slot < a.nsamp) {
                s_rec[threadIdx.x][0] = make_uint4(__float_as_uint(ov.x), __float_as_uint(ov.y),
                                                   __float_as_uint(sg.ft), __float_as_uint(sg.fh));
                s_rec[threadIdx.x][1] = make_uint4(__float_as_uint(sg.fw), sid0 + (uint32_t)p,
                                                   (uint32_t)qrow_bytes, (uint32_t)(qrow_bytes >> 32));
                my_slot = slot;
            }
        }
        s_slot[threadIdx.x] = my_slot;
        wave_lds_sync();
        // Each record is written by a pair of neighbouring lanes of its group,
        // one 16-byte half each, so that a record costs one 32-byte write
        // request rather than two: in two rounds, lanes (2i, 2i+1) write the
        // record of the group's lane (L/2)*round + i. (With one lane per
        // group, that lane writes both halves.)
        if constexpr (L >= 2) {
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int src = (int)threadIdx.x - li + r * (L / 2) + (li >> 1);
                const uint32_t sl = s_slot[src];
                if (sl != kNoSlot) reinterpret_cast<uint4*>(a.rec + sl)[li & 1] = s_rec[src][li & 1];
            }
        } else if (my_slot != kNoSlot) {
            reinterpret_cast<uint4*>(a.rec + my_slot)[0] = s_rec[threadIdx.x][0];
            reinterpret_cast<uint4*>(a.rec + my_slot)[1] = s_rec[threadIdx.x][1];
        }
    }
    Frag8<T> dqf;
    dqf.from_f32(dq);
    dqf.store(reinterpret_cast<T*>(a.dq) + tok * C + row_off);
}

// ---------------------------------------------------------------------------
// 4. deterministic mode: sort the records of every bucket by sample number.
//
// Bitonic network in the form whose comparators all put the smaller key at
// the lower index (a "flip" stage, then half-cleaners), so a bucket of n keys
// sorts as if padded with +infinity up to a power of two while only the real
// n entries are touched: a comparator whose upper index is >= n would leave
// its pair unchanged and is skipped. Sample numbers are distinct.
// ---------------------------------------------------------------------------
template <typename Swap, typename Sync>
__device__ __forceinline__ void bitonic_sort(uint32_t n, uint32_t tid, uint32_t nthr, Swap cmpswap, Sync sync) {
    uint64_t npad = 1;  // 64-bit: a bucket may hold up to 2^32 - 1 entries
    while (npad < n) npad <<= 1;
    const uint64_t pairs = npad / 2;
    for (uint64_t k = 2; k <= npad; k <<= 1) {
        const uint64_t half = k >> 1;
        for (uint64_t i = tid; i < pairs; i += nthr) {
            const uint64_t blk = (i / half) * k, off = i % half;
            const uint64_t lo = blk + off, hi = blk + k - 1 - off;
            if (hi < n) cmpswap(lo, hi);
        }
        sync();
        for (uint64_t j = half >> 1; j >= 1; j >>= 1) {
            for (uint64_t i = tid; i < pairs; i += nthr) {
                const uint64_t lo = (i / j) * 2 * j + (i % j), hi = lo + j;
                if (hi < n) cmpswap(lo, hi);
            }
            sync();
        }
    }
}

struct BlockSync {
    __device__ __forceinline__ void operator()() const { __syncthreads(); }
};

// (sample number << 32 | position) keys in LDS, compare-exchanged.
struct LdsKeySwap {
    uint64_t* key;
    __device__ __forceinline__ void operator()(uint64_t lo, uint64_t hi) const {
        const uint64_t x = key[lo], y = key[hi];
        if (x > y) { key[lo] = y; key[hi] = x; }
    }
};

// Whole 32-byte records in global memory, compared by sample number.
struct GlobalRecSwap {
    uint4* rec;  // two uint4 per record; the sample number is word 5
    __device__ __forceinline__ void operator()(uint64_t lo, uint64_t hi) const {
        const uint4 a1 = rec[2 * hi + 1];
        const uint4 b1 = rec[2 * lo + 1];
        if (b1.y > a1.y) {
            const uint4 a0 = rec[2 * hi], b0 = rec[2 * lo];
            rec[2 * lo] = a0; rec[2 * lo + 1] = a1;
            rec[2 * hi] = b0; rec[2 * hi + 1] = b1;
        }
    }
};

// Buckets of 2 to kRankSortMax records (nearly all of them: a bucket holds P
// records on average): one wave per block walks kSortBucketsPerBlock
// consecutive buckets. Lane l holds records l and l + 64 in registers and puts
// their sample numbers in LDS; the rank of a record is the number of sample
// numbers in the bucket below its own (they are distinct), and each lane
// writes its records to their ranks (all reads precede all writes, so the
// permutation is done in place). The next bucket's records are requested
// before the current bucket is ranked.
constexpr uint32_t kRankSortMax = 128;

struct RankPair {
    uint4 a0, a1, b0, b1;  // records lane and lane + 64 (word 5 = a1.y / b1.y is the sample number)
};

__device__ __forceinline__ void rank_fetch(const uint4* grec, uint32_t s, uint32_t n, uint32_t lane, RankPair& r) {
    if (n < 2 || n > kRankSortMax) return;
    if (lane < n) {
        r.a0 = grec[2 * ((uint64_t)s + lane)];
        r.a1 = grec[2 * ((uint64_t)s + lane) + 1];
    }
    if (lane + 64 < n) {
        r.b0 = grec[2 * ((uint64_t)s + lane + 64)];
        r.b1 = grec[2 * ((uint64_t)s + lane + 64) + 1];
    }
}

__global__ void __launch_bounds__(64) dsa3d_sort_rank_kernel(const uint32_t* start, uint32_t ncell, SampleRec* rec) {
    __shared__ __attribute__((aligned(16))) uint32_t skey[kRankSortMax];
    const uint32_t c0 = blockIdx.x * kSortBucketsPerBlock;
    const uint32_t nb = min(ncell - c0, (uint32_t)kSortBucketsPerBlock);
    uint4* grec = reinterpret_cast<uint4*>(rec);
    const uint32_t lane = threadIdx.x;
    // bucket starts of the block: lane l holds start[c0 + l], and one more at the end
    const uint32_t my_start = lane <= nb ? start[c0 + lane] : 0u;
    const uint32_t end_start = start[c0 + nb];
    auto bucket = [&](uint32_t i, uint32_t& s0, uint32_t& n) {
        s0 = (uint32_t)__shfl((int)my_start, (int)i, 64);
        const uint32_t s1 = i + 1 < 64 ? (uint32_t)__shfl((int)my_start, (int)(i + 1), 64) : end_start;
        n = (i + 1 == nb ? end_start : s1) - s0;
    };
    RankPair cur{}, nxt{};
    uint32_t s, n;
    bucket(0, s, n);
    rank_fetch(grec, s, n, lane, cur);
    for (uint32_t i = 0; i < nb; ++i) {
        uint32_t sn = 0, nn = 0;
        if (i + 1 < nb) {
            bucket(i + 1, sn, nn);
            rank_fetch(grec, sn, nn, lane, nxt);
        }
        if (n >= 2 && n <= kRankSortMax) {
            const bool ha = lane < n, hb = lane + 64 < n;
            // slots past the bucket hold the largest key, which no sample number reaches
            skey[lane] = ha ? cur.a1.y : 0xffffffffu;
            skey[lane + 64] = hb ? cur.b1.y : 0xffffffffu;
            wave_lds_sync();
            uint32_t ra = 0, rb = 0;
            const uint4* k4 = reinterpret_cast<const uint4*>(skey);
            for (uint32_t k = 0; k < (n + 3) / 4; ++k) {
                const uint4 q = k4[k];
                ra += (q.x < cur.a1.y ? 1u : 0u) + (q.y < cur.a1.y ? 1u : 0u) + (q.z < cur.a1.y ? 1u : 0u) +
                      (q.w < cur.a1.y ? 1u : 0u);
                rb += (q.x < cur.b1.y ? 1u : 0u) + (q.y < cur.b1.y ? 1u : 0u) + (q.z < cur.b1.y ? 1u : 0u) +
                      (q.w < cur.b1.y ? 1u : 0u);
            }
            if (ha) {
                grec[2 * ((uint64_t)s + ra)] = cur.a0;
                grec[2 * ((uint64_t)s + ra) + 1] = cur.a1;
            }
            if (hb) {
                grec[2 * ((uint64_t)s + rb)] = cur.b0;
                grec[2 * ((uint64_t)s + rb) + 1] = cur.b1;
            }
            wave_lds_sync();  // every lane has read the keys before the next bucket writes them
        }
        cur = nxt;
        s = sn;
        n = nn;
    }
}

// Buckets of kRankSortMax + 1 to kWaveSortMax records: one wave per block;
// the block walks kSortBucketsPerBlock consecutive buckets (skipping the
// smaller ones). A bucket is held in registers (lane
// l holds records l, l+64, ...), its (sample number, position) keys are
// sorted in LDS, and each lane then writes the records it holds straight to
// their sorted positions (all reads precede all writes, so the permutation is
// done in place). Larger buckets are queued in `large` ([0] = count,
// [1..cap] = bucket numbers) for the next kernel.
__global__ void __launch_bounds__(64) dsa3d_sort_small_kernel(const uint32_t* start, uint32_t ncell, SampleRec* rec,
                                                              uint32_t* large, uint32_t large_cap) {
    constexpr int kPer = kWaveSortMax / 64;  // records per lane
    __shared__ uint64_t skey[kWaveSortMax];
    __shared__ uint16_t srank[kWaveSortMax];
    const uint32_t c0 = blockIdx.x * kSortBucketsPerBlock;
    const uint32_t c1 = min(ncell, c0 + kSortBucketsPerBlock);
    uint4* grec = reinterpret_cast<uint4*>(rec);
    const uint32_t lane = threadIdx.x;
    for (uint32_t c = c0; c < c1; ++c) {
        const uint32_t s = start[c], n = start[c + 1] - s;
        if (n <= kRankSortMax) continue;
        if (n > kWaveSortMax) {
            if (lane == 0) {
                const uint32_t slot = atomicAdd(large, 1u);
                if (slot < large_cap) large[1 + slot] = c;
            }
            continue;
        }
        uint4 r0[kPer], r1[kPer];
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            const uint32_t i = lane + 64u * k;
            if (i < n) {
                r0[k] = grec[2 * ((uint64_t)s + i)];
                r1[k] = grec[2 * ((uint64_t)s + i) + 1];
                skey[i] = ((uint64_t)r1[k].y << 32) | i;
            }
        }
        __syncthreads();
        bitonic_sort(n, lane, 64, LdsKeySwap{skey}, BlockSync());
        for (uint32_t i = lane; i < n; i += 64) srank[(uint32_t)skey[i]] = (uint16_t)i;
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            const uint32_t i = lane + 64u * k;
            if (i < n) {
                const uint64_t dst = (uint64_t)s + srank[i];
                grec[2 * dst] = r0[k];
                grec[2 * dst + 1] = r1[k];
            }
        }
        __syncthreads();
    }
}

// Buckets queued by the previous kernel, sorted in place in global memory by
// one 1024-thread block each (same network). Only an offset field that sends
// hundreds of samples into one cell takes this path.
__global__ void __launch_bounds__(1024) dsa3d_sort_large_kernel(const uint32_t* start, SampleRec* rec,
                                                                const uint32_t* large, uint32_t large_cap) {
    const uint32_t count = min(large[0], large_cap);
    for (uint32_t item = blockIdx.x; item < count; item += gridDim.x) {
        const uint32_t c = large[1 + item];
        const uint32_t s = start[c], n = start[c + 1] - s;
        bitonic_sort(n, threadIdx.x, blockDim.x, GlobalRecSwap{reinterpret_cast<uint4*>(rec + s)}, BlockSync());
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// 5. key kernel: one task = four keys, two frames by two tokens along w
//    ((t, w), (t, w+1), (t+1, w), (t+1, w+1), with t and w even)
//
// Key y takes the records of the buckets of base cells y - c. For the group
// those are the cells of frames t-1 .. t+1, rows h-1 and h, and columns
// w-1 .. w+1: 18 buckets, against 32 for four keys taken one by one. A cell
// reaches the keys whose offset from it is a corner (0 or 1 on each axis):
// frame t-1 only the keys of frame t, frame t+1 only those of frame t+1, and
// frame t both; likewise along w. The group walks its buckets class by class
// (frame class, then column class; within a class its two rows, then bucket
// order), so each record and its query and output-gradient rows are read once
// for every key they reach, and each entry updates only the keys its class
// reaches (1.8 on average).
// ---------------------------------------------------------------------------
constexpr int kQuadBuckets = 18;

template <int N>
using IntC = std::integral_constant<int, N>;

// Rows of 128 channels or more take four entries per step (eight row loads in
// flight) at three waves per SIMD: a 3-head pass at 1080p runs in 60 ms, against
// 65 ms with two entries at four waves and 67 ms with eight at two. Narrower
// rows take two entries per step, bf16 rows of 64 channels at four waves (the
// 720p pass: 8.5 ms, against 9.1 ms with four entries and 11.9 ms at two waves).
template <int D>
constexpr int key_entries_per_step() { return D >= 128 ? 4 : 2; }
template <typename T, int D>
constexpr int key_kernel_waves() { return D >= 128 ? 3 : std::is_same<T, bf16_t>::value && D == 64 ? 4 : 1; }

template <typename T, int D>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(key_kernel_waves<T, D>())))
dsa3d_bwd_key_kernel(BwdArgs a) {
    constexpr int L = D / 8;
    const int g = threadIdx.x / L;
    const int li = threadIdx.x % L;
    int64_t bh;
    int32_t tp, h, wb;
    TaskGrid gp = a.g;
    gp.T = (a.g.T + 1) / 2;  // the block order walks pairs of frames
    block_coords(gp, a.ord, logical_block(blockIdx.x, gridDim.x, a.ord.chunk), bh, tp, h, wb);
    const int32_t t = 2 * tp;
    const int32_t w = wb + 2 * g;
    if (w >= a.g.W) return;  // no block-wide barrier below
    const bool right = w + 1 < a.g.W, late = t + 1 < a.g.T;  // the group's second token along w / in t exists
    const int32_t b = (int32_t)(bh / a.g.nheads);
    const int32_t eta = a.g.head0 + (int32_t)(bh - (int64_t)b * a.g.nheads);
    const int64_t tok = (((int64_t)b * a.g.T + t) * a.g.H + h) * a.g.W + w;
    const int64_t C = (int64_t)a.g.heads * D;
    const int64_t row_off = (int64_t)eta * D + li * 8;
    const uint4* rec = reinterpret_cast<const uint4*>(a.rec);

    // The group's buckets, class by class: bucket (it*3 + j)*2 + ch is the cell
    // of frame t-1+it, row h-ch, column w-1+j; start and size kept in LDS.
    __shared__ uint32_t s_bs[256 / L][kQuadBuckets], s_n[256 / L][kQuadBuckets];
    __shared__ float4 s_coef[256][2];  // per entry: (scale*ds*w, a*w) of up to four keys
    __shared__ uint2 s_row[256];       // byte offset of the query's row
    uint32_t* bs = s_bs[g];
    uint32_t* bn = s_n[g];
    float4 (*coef)[2] = s_coef + (threadIdx.x - li);
    uint2* row = s_row + (threadIdx.x - li);
#pragma unroll
    for (int i = 0; i < kQuadBuckets; ++i) {
        const int it = i / 6, j = (i >> 1) % 3, ch = i & 1;
        uint32_t s0 = 0u, n = 0u;
        if ((it < 2 || late) && (j < 2 || right)) {
            const uint32_t cell = cell_index(a.g, bh, t - 1 + it, h - ch, w - 1 + j);
            s0 = a.start[cell];
            n = a.start[cell + 1] - s0;
        }
        if (li == 0) { bs[i] = s0; bn[i] = n; }
    }
    const char* Qc = reinterpret_cast<const char*>(reinterpret_cast<const T*>(a.q) + row_off);
    const char* Gc = reinterpret_cast<const char*>(reinterpret_cast<const T*>(a.dout) + row_off);
    float ak[4][8], av[4][8];
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int e = 0; e < 8; ++e) { ak[k][e] = 0.f; av[k][e] = 0.f; }

    // One class: the two buckets of frame class IT and column class J reach the
    // keys dt in [IT == 2, IT != 0] and dw in [J == 2, J != 0] of the group.
    auto run = [&](auto it_c, auto j_c) {
        constexpr int IT = decltype(it_c)::value, J = decltype(j_c)::value;
        constexpr int T0 = IT == 2 ? 1 : 0, T1 = IT == 0 ? 0 : 1, W0 = J == 2 ? 1 : 0, W1 = J == 0 ? 0 : 1;
        constexpr int i0 = (IT * 3 + J) * 2;
        wave_lds_sync();  // the bucket table is written; the previous class's entries have been read
        const uint32_t n0 = bn[i0], N = n0 + bn[i0 + 1];
        const uint32_t b0 = bs[i0], b1 = bs[i0 + 1];
        for (uint32_t k0 = 0; k0 < N; k0 += L) {
            const uint32_t n = min((uint32_t)L, N - k0);
            wave_lds_sync();  // the previous chunk has been read
            if ((uint32_t)li < n) {
                const uint32_t k = k0 + li;
                const int ch = k < n0 ? 0 : 1;
                const uint32_t e = ch ? b1 + (k - n0) : b0 + k;
                const uint4 r0 = rec[2 * (uint64_t)e], r1 = rec[2 * (uint64_t)e + 1];
                const float ft = __uint_as_float(r0.z), fh = __uint_as_float(r0.w), fw = __uint_as_float(r1.x);
                const float ck = __uint_as_float(r0.x), cv = __uint_as_float(r0.y);
                const float wh = ch ? fh : 1.0f - fh;
                float c8[8];
#pragma unroll
                for (int q = 0; q < 4; ++q) {  // key (dt, dw): corner (dt + 1 - IT, ch, dw + 1 - J)
                    const int dt = q >> 1, dw = q & 1;
                    float wt = 0.0f;
                    if (dt >= T0 && dt <= T1 && dw >= W0 && dw <= W1) {
                        const int ct = dt + 1 - IT, cw = dw + 1 - J;
                        wt = ((ct ? ft : 1.0f - ft) * wh) * (cw ? fw : 1.0f - fw);
                    }
                    c8[2 * q] = ck * wt;
                    c8[2 * q + 1] = cv * wt;
                }
                coef[li][0] = make_float4(c8[0], c8[1], c8[2], c8[3]);
                coef[li][1] = make_float4(c8[4], c8[5], c8[6], c8[7]);
                row[li] = make_uint2(r1.z, r1.w);
            }
            wave_lds_sync();
            auto add = [&](const Frag8<T>& qx, const Frag8<T>& gx, const float4& c0, const float4& c1) {
                const float cc[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int dt = q >> 1, dw = q & 1;
                    if (dt >= T0 && dt <= T1 && dw >= W0 && dw <= W1) {
                        qx.axpy(cc[2 * q], ak[q]);
                        gx.axpy(cc[2 * q + 1], av[q]);
                    }
                }
            };
            uint32_t j = 0;
            for (; key_entries_per_step<D>() == 4 && j + 3 < n; j += 4) {  // eight row loads in flight
                const uint2 ra = row[j], rb = row[j + 1], rc = row[j + 2], rd = row[j + 3];
                const uint64_t oa = ((uint64_t)ra.y << 32) | ra.x, ob = ((uint64_t)rb.y << 32) | rb.x;
                const uint64_t oc = ((uint64_t)rc.y << 32) | rc.x, od = ((uint64_t)rd.y << 32) | rd.x;
                Frag8<T> qa, ga, qb, gb, qc, gc, qd, gd;
                qa.load(reinterpret_cast<const T*>(Qc + oa));
                ga.load(reinterpret_cast<const T*>(Gc + oa));
                qb.load(reinterpret_cast<const T*>(Qc + ob));
                gb.load(reinterpret_cast<const T*>(Gc + ob));
                qc.load(reinterpret_cast<const T*>(Qc + oc));
                gc.load(reinterpret_cast<const T*>(Gc + oc));
                qd.load(reinterpret_cast<const T*>(Qc + od));
                gd.load(reinterpret_cast<const T*>(Gc + od));
                add(qa, ga, coef[j][0], coef[j][1]);
                add(qb, gb, coef[j + 1][0], coef[j + 1][1]);
                add(qc, gc, coef[j + 2][0], coef[j + 2][1]);
                add(qd, gd, coef[j + 3][0], coef[j + 3][1]);
            }
            for (; j + 1 < n; j += 2) {  // two entries per step: four row loads in flight
                const uint2 ra = row[j], rb = row[j + 1];
                const uint64_t oa = ((uint64_t)ra.y << 32) | ra.x, ob = ((uint64_t)rb.y << 32) | rb.x;
                Frag8<T> qa, ga, qb, gb;
                qa.load(reinterpret_cast<const T*>(Qc + oa));
                ga.load(reinterpret_cast<const T*>(Gc + oa));
                qb.load(reinterpret_cast<const T*>(Qc + ob));
                gb.load(reinterpret_cast<const T*>(Gc + ob));
                add(qa, ga, coef[j][0], coef[j][1]);
                add(qb, gb, coef[j + 1][0], coef[j + 1][1]);
            }
            if (j < n) {
                const uint2 ra = row[j];
                const uint64_t oa = ((uint64_t)ra.y << 32) | ra.x;
                Frag8<T> qa, ga;
                qa.load(reinterpret_cast<const T*>(Qc + oa));
                ga.load(reinterpret_cast<const T*>(Gc + oa));
                add(qa, ga, coef[j][0], coef[j][1]);
            }
        }
    };
    run(IntC<0>{}, IntC<0>{}); run(IntC<0>{}, IntC<1>{}); run(IntC<0>{}, IntC<2>{});
    run(IntC<1>{}, IntC<0>{}); run(IntC<1>{}, IntC<1>{}); run(IntC<1>{}, IntC<2>{});
    run(IntC<2>{}, IntC<0>{}); run(IntC<2>{}, IntC<1>{}); run(IntC<2>{}, IntC<2>{});

    const int64_t HW = (int64_t)a.g.H * a.g.W;
    Frag8<T> f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int dt = q >> 1, dw = q & 1;
        if ((dt && !late) || (dw && !right)) continue;
        const int64_t tq = tok + dt * HW + dw;
        f.from_f32(ak[q]);
        f.store(reinterpret_cast<T*>(a.dk) + tq * C + row_off);
        f.from_f32(av[q]);
        f.store(reinterpret_cast<T*>(a.dv) + tq * C + row_off);
    }
}

// ---------------------------------------------------------------------------
// Host side: workspace layout and launch sequence
// ---------------------------------------------------------------------------
namespace {

struct BwdLayout {
    uint64_t ncell, nsamp, nscan, large_cap;
    size_t off_cnt, off_start, off_bsum, off_large, off_rec, total;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// The tiled count's histogram: the window's reach per axis plus up to 4 cells
// of offset margin, as much as fits in the LDS histogram (none: the untiled
// count kernel is used).
bool count_tile(const dsa3d_desc& d, CountTile& ct) {
    const int64_t reach_t = (int64_t)(d.kt - 1) / 2 * d.dil_t, reach_h = (int64_t)(d.kh - 1) / 2 * d.dil_h,
                  reach_w = (int64_t)(d.kw - 1) / 2 * d.dil_w;
    for (int extra = 4; extra >= 0; --extra) {
        const int64_t mt = reach_t + extra, mh = reach_h + extra, mw = reach_w + extra;
        const int64_t RT = kCtT + 2 * mt + 1, RH = kCtH + 2 * mh + 1, RW = kCtW + 2 * mw + 1;
        if (RT * RH * RW <= kCountLdsCells) {
            ct.mt = (int32_t)mt; ct.mh = (int32_t)mh; ct.mw = (int32_t)mw;
            ct.RT = (int32_t)RT; ct.RH = (int32_t)RH; ct.RW = (int32_t)RW;
            ct.ntt = (int32_t)((d.T + kCtT - 1) / kCtT);
            ct.nth = (int32_t)((d.H + kCtH - 1) / kCtH);
            ct.ntw = (int32_t)((d.W + kCtW - 1) / kCtW);
            return true;
        }
    }
    return false;
}

bool bwd_layout(const dsa3d_desc& d, int64_t nh, BwdLayout& L) {
    const uint64_t ntok = (uint64_t)(d.B * d.T * d.H * d.W);
    const uint64_t cells_per_bh = (uint64_t)(d.T + 1) * (uint64_t)(d.H + 1) * (uint64_t)(d.W + 1);
    L.ncell = (uint64_t)nh * (uint64_t)d.B * cells_per_bh;
    L.nsamp = (uint64_t)nh * ntok * (uint64_t)d.P;
    if (L.ncell + 1 >= (uint64_t(1) << 32) || L.nsamp >= (uint64_t(1) << 32)) return false;
    L.nscan = (L.ncell + kScanChunk - 1) / kScanChunk;
    L.large_cap = L.nsamp / (kWaveSortMax + 1) + 1;
    size_t o = 0;
    L.off_cnt = o;   o += align256(L.ncell * 4);
    L.off_start = o; o += align256((L.ncell + 1) * 4);
    L.off_bsum = o;  o += align256(L.nscan * 4 + 4);
    L.off_large = o; o += align256((L.large_cap + 1) * 4);
    L.off_rec = o;   o += align256(L.nsamp * sizeof(SampleRec));
    L.total = o;
    return true;
}

template <typename T, int D>
hipError_t bwd_query_t(const BwdArgs& a, int64_t nb, hipStream_t s) {
    LaunchScope ls(DSA3D_K_BWD_QUERY, s);
    hipLaunchKernelGGL((dsa3d_bwd_query_kernel<T, D>), dim3((unsigned)nb), dim3(256), 0, s, a);
    return hipGetLastError();
}
template <int D> hipError_t bwd_query_f32(const BwdArgs& a, int64_t nb, hipStream_t s) { return bwd_query_t<float, D>(a, nb, s); }
template <int D> hipError_t bwd_query_bf16(const BwdArgs& a, int64_t nb, hipStream_t s) { return bwd_query_t<bf16_t, D>(a, nb, s); }

template <typename T, int D>
hipError_t bwd_key_t(const BwdArgs& a, int64_t nb, hipStream_t s) {
    LaunchScope ls(DSA3D_K_BWD_KEY, s);
    hipLaunchKernelGGL((dsa3d_bwd_key_kernel<T, D>), dim3((unsigned)nb), dim3(256), 0, s, a);
    return hipGetLastError();
}
template <int D> hipError_t bwd_key_f32(const BwdArgs& a, int64_t nb, hipStream_t s) { return bwd_key_t<float, D>(a, nb, s); }
template <int D> hipError_t bwd_key_bf16(const BwdArgs& a, int64_t nb, hipStream_t s) { return bwd_key_t<bf16_t, D>(a, nb, s); }

}  // namespace

size_t bwd_workspace_bytes(const dsa3d_desc& d, int64_t nheads) {
    BwdLayout L;
    if (nheads < 1 || !bwd_layout(d, nheads, L)) return 0;
    return L.total;
}

int64_t bwd_heads_per_pass(const dsa3d_desc& d, size_t ws_bytes) {
    int64_t lo = 0, hi = d.heads;  // largest nh in [1, heads] that fits, or 0
    while (lo < hi) {
        const int64_t mid = (lo + hi + 1) / 2;
        const size_t need = bwd_workspace_bytes(d, mid);
        if (need != 0 && need <= ws_bytes) lo = mid; else hi = mid - 1;
    }
    return lo;
}

hipError_t launch_backward(const dsa3d_desc& d, const void* q, const void* k, const void* v, const void* off,
                           const void* o, const float* lse, const void* dout, void* dq, void* dk, void* dv,
                           void* doff, void* ws, size_t ws_bytes, hipStream_t s) {
    const int64_t ntok = d.B * d.T * d.H * d.W;
    if (ntok == 0) return hipSuccess;
    const int64_t chunk = bwd_heads_per_pass(d, ws_bytes);
    if (chunk < 1) return hipErrorInvalidValue;
    const bool f32 = d.dtype == DSA3D_F32;
    const BlockOrder ord = make_block_order(d, attn_tokens_per_block(d.head_dim), kQuerySupertile, "DSA3D_ORDER_Q");
    dsa3d_desc dpair = d;
    dpair.T = (d.T + 1) / 2;
    const BlockOrder kord = make_block_order(dpair, 2 * attn_tokens_per_block(d.head_dim), kKeySupertile,
                                             "DSA3D_ORDER_KEY");
    hipError_t e;
    for (int64_t h0 = 0; h0 < d.heads; h0 += chunk) {
        const int32_t nh = (int32_t)std::min<int64_t>(chunk, d.heads - h0);
        BwdLayout L;
        bwd_layout(d, nh, L);
        char* base = static_cast<char*>(ws);
        BwdArgs a{};
        a.q = q; a.k = k; a.v = v; a.off = off; a.o = o; a.dout = dout; a.lse = lse;
        a.dq = dq; a.doff = doff; a.dk = dk; a.dv = dv;
        a.cnt = reinterpret_cast<uint32_t*>(base + L.off_cnt);
        a.start = reinterpret_cast<uint32_t*>(base + L.off_start);
        a.rec = reinterpret_cast<SampleRec*>(base + L.off_rec);
        a.nsamp = (uint32_t)L.nsamp;
        a.g = make_task_grid(d, (int32_t)h0, nh);
        a.ord = ord;
        a.P = d.P;
        a.scale = logit_scale(d);
        a.win = make_window(d);
        uint32_t* bsum = reinterpret_cast<uint32_t*>(base + L.off_bsum);
        uint32_t* large = reinterpret_cast<uint32_t*>(base + L.off_large);
        const uint32_t ncell = (uint32_t)L.ncell;
        const int64_t nblocks = ord.nblk_bh * d.B * nh;

        // 1. bucket counts
        if ((e = fill_zero(a.cnt, L.ncell * 4, s)) != hipSuccess) return e;
        if ((e = fill_zero(large, 4, s)) != hipSuccess) return e;
        {
            LaunchScope ls(DSA3D_K_BWD_COUNT, s);
            CountTile ct;
            if (count_tile(d, ct)) {
                const int64_t nb = (int64_t)d.B * nh * ct.ntt * ct.nth * ct.ntw;
                if (f32) hipLaunchKernelGGL(dsa3d_bwd_count_tiled_kernel<float>, dim3((unsigned)nb), dim3(256), 0, s, a, ct);
                else hipLaunchKernelGGL(dsa3d_bwd_count_tiled_kernel<bf16_t>, dim3((unsigned)nb), dim3(256), 0, s, a, ct);
            } else {
                const unsigned gb = grid_for((int64_t)L.nsamp, 256, 1 << 16);
                if (f32) hipLaunchKernelGGL(dsa3d_bwd_count_kernel<float>, dim3(gb), dim3(256), 0, s, a);
                else hipLaunchKernelGGL(dsa3d_bwd_count_kernel<bf16_t>, dim3(gb), dim3(256), 0, s, a);
            }
        }
        if ((e = hipGetLastError()) != hipSuccess) return e;
        // 2. bucket starts, which also become the fill cursors
        {
            LaunchScope ls(DSA3D_K_BWD_SCAN, s);
            hipLaunchKernelGGL(dsa3d_scan_sums_kernel, dim3((unsigned)L.nscan), dim3(kScanThreads), 0, s, a.cnt, ncell,
                               bsum);
            hipLaunchKernelGGL(dsa3d_scan_top_kernel, dim3(1), dim3(1024), 0, s, bsum, (uint32_t)L.nscan, a.start, ncell);
            hipLaunchKernelGGL(dsa3d_scan_apply_kernel, dim3((unsigned)L.nscan), dim3(kScanThreads), 0, s, a.cnt,
                               ncell, bsum, a.start);
        }
        if ((e = hipGetLastError()) != hipSuccess) return e;
        // 3. dq, doffsets and the sample records
        if (f32) { DSA3D_DISPATCH_D_E(d.head_dim, bwd_query_f32, e, a, nblocks, s); }
        else { DSA3D_DISPATCH_D_E(d.head_dim, bwd_query_bf16, e, a, nblocks, s); }
        if (e != hipSuccess) return e;
        // 4. fixed summation order
        if (d.deterministic) {
            LaunchScope ls(DSA3D_K_BWD_SORT, s);
            const unsigned nblk = (unsigned)((L.ncell + kSortBucketsPerBlock - 1) / kSortBucketsPerBlock);
            hipLaunchKernelGGL(dsa3d_sort_rank_kernel, dim3(nblk), dim3(64), 0, s, a.start, ncell, a.rec);
            hipLaunchKernelGGL(dsa3d_sort_small_kernel, dim3(nblk), dim3(64), 0, s, a.start, ncell, a.rec, large,
                               (uint32_t)L.large_cap);
            hipLaunchKernelGGL(dsa3d_sort_large_kernel, dim3(256), dim3(1024), 0, s, a.start, a.rec, large,
                               (uint32_t)L.large_cap);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        // 5. dk, dv (two keys per task)
        a.ord = kord;
        const int64_t kblocks = kord.nblk_bh * d.B * nh;
        if (f32) { DSA3D_DISPATCH_D_E(d.head_dim, bwd_key_f32, e, a, kblocks, s); }
        else { DSA3D_DISPATCH_D_E(d.head_dim, bwd_key_bf16, e, a, kblocks, s); }
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace dsa3d
