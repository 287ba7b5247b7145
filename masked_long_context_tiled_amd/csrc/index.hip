// Tile index construction on the device.
//
// Dense masks: every (query tile, key tile) is classified EMPTY / PARTIAL / FULL from
// the column-interval descriptor, then the non-empty tiles are listed per query tile
// (CSR, walked by the forward) and per key tile (CSC, walked by the backward), in
// ascending order, each entry (tile << 1) | is_full. A launch order sorts the work
// items by descending list length so the longest run first.
//
// Block-sparse masks: the keep matrix is listed the same way, per (head, query block)
// row and per (KV head, key block) column.
#include "common.h"

namespace mlct {

enum : uint8_t { CLS_EMPTY = 0, CLS_PARTIAL = 1, CLS_FULL = 2 };

// The forward and backward halves of the index are built by the same launches: each
// kernel below takes two jobs and splits its grid between them (the first a.blocks
// workgroups run job a, the rest job b), so building an index takes five launches.

struct ClassifyJob {
    int BM, BN, nqt, nkt;
    uint8_t* cls;
    int blocks;
};

// One thread per tile. Threads of a wave share the key tile (consecutive query tiles),
// so the descriptor reads are broadcast.
__global__ void classify_kernel(const int4* __restrict__ desc, int T, ClassifyJob a, ClassifyJob b) {
    const bool second = (int)blockIdx.x >= a.blocks;
    const ClassifyJob j = second ? b : a;
    const long t = (long)(second ? blockIdx.x - a.blocks : blockIdx.x) * blockDim.x + threadIdx.x;
    if (t >= (long)j.nqt * j.nkt) return;
    const int kt = (int)(t / j.nqt), qt = (int)(t % j.nqt);
    const int r0 = qt * j.BM, r1 = min(T, r0 + j.BM);
    const int c0 = kt * j.BN, c1 = min(T, c0 + j.BN);
    const int rows = r1 - r0;
    bool any = false, all = true;
    // unrolled so that several descriptor reads are in flight (the loop is latency-bound)
#pragma unroll 8
    for (int c = c0; c < c1; ++c) {
        const int4 d = desc[c];
        const int n0 = max(0, min(d.y, r1) - max(d.x, r0));
        const int n1 = max(0, min(d.w, r1) - max(d.z, r0));
        const int n = n0 + n1;
        any |= n > 0;
        all &= n == rows;
    }
    j.cls[(size_t)qt * j.nkt + kt] = any ? (all ? CLS_FULL : CLS_PARTIAL) : CLS_EMPTY;
}

// Lists: list l has `len` elements; element m of list l is at
//   src[(l / div) * s_hi + (l % div) * s_lo + m * s_m].
struct ListGeom {
    int nlists, len, div;
    long s_hi, s_lo, s_m;
};

// One list job: the source map, its geometry, the row pointers and entries written, whether
// entries carry the FULL bit, and the workgroups (4 waves each, one wave per list) it takes.
struct ListJob {
    const uint8_t* src;
    ListGeom g;
    int* ptr;
    int* ent;
    int tag_full;
    int blocks;
};

__device__ __forceinline__ size_t elem_addr(const ListGeom& g, int l, int m) {
    return (size_t)((long)(l / g.div) * g.s_hi + (long)(l % g.div) * g.s_lo + (long)m * g.s_m);
}

// One wave per list: count non-zero elements into ptr[l + 1] (ptr[0] = 0).
__global__ void list_count_kernel(ListJob a, ListJob b) {
    const bool second = (int)blockIdx.x >= a.blocks;
    const ListJob j = second ? b : a;
    const int wave = (int)(((second ? blockIdx.x - a.blocks : blockIdx.x) * blockDim.x + threadIdx.x) >> 6);
    const int lane = threadIdx.x & 63;
    if (wave >= j.g.nlists) return;
    int count = 0;
    for (int m0 = 0; m0 < j.g.len; m0 += 64) {
        const int m = m0 + lane;
        const bool nz = m < j.g.len && j.src[elem_addr(j.g, wave, m)] != 0;
        count += __popcll(__ballot(nz));
    }
    if (lane == 0) {
        j.ptr[wave + 1] = count;
        if (wave == 0) j.ptr[0] = 0;
    }
}

// One wave per list: write the indices of non-zero elements in ascending order,
// (m << 1) | (value == FULL) when tag_full, else m.
__global__ void list_fill_kernel(ListJob a, ListJob b) {
    const bool second = (int)blockIdx.x >= a.blocks;
    const ListJob j = second ? b : a;
    const int wave = (int)(((second ? blockIdx.x - a.blocks : blockIdx.x) * blockDim.x + threadIdx.x) >> 6);
    const int lane = threadIdx.x & 63;
    if (wave >= j.g.nlists) return;
    int base = j.ptr[wave];
    const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int m0 = 0; m0 < j.g.len; m0 += 64) {
        const int m = m0 + lane;
        const uint8_t v = m < j.g.len ? j.src[elem_addr(j.g, wave, m)] : 0;
        const unsigned long long bl = __ballot(v != 0);
        if (v != 0) j.ent[base + __popcll(bl & below)] = j.tag_full ? ((m << 1) | (v == CLS_FULL)) : m;
        base += __popcll(bl);
    }
}

// In-place inclusive prefix sum of a[1..n] (a[0] = 0), one workgroup of 1024 threads per
// job: workgroup 0 scans job a's pointers, workgroup 1 job b's.
__global__ __launch_bounds__(1024) void scan_kernel(ListJob ja, ListJob jb) {
    __shared__ int part[1024];
    int* a = blockIdx.x == 0 ? ja.ptr : jb.ptr;
    const int n = blockIdx.x == 0 ? ja.g.nlists : jb.g.nlists;
    const int t = threadIdx.x;
    const int chunk = (n + 1023) / 1024;
    const int lo = 1 + t * chunk, hi = min(n + 1, lo + chunk);
    int s = 0;
    for (int i = lo; i < hi; ++i) s += a[i];
    part[t] = s;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
        const int v = t >= off ? part[t - off] : 0;
        __syncthreads();
        part[t] += v;
        __syncthreads();
    }
    int run = t > 0 ? part[t - 1] : 0;
    for (int i = lo; i < hi; ++i) {
        run += a[i];
        a[i] = run;
    }
}

// order[rank] = i, ranks by descending list length, ties by ascending index (lists of up
// to 65536 work items; longer ones keep the identity order).
struct OrderJob {
    const int* ptr;
    int n;
    int* order;
    int blocks;
};
__global__ void order_kernel(OrderJob a, OrderJob b) {
    __shared__ int cnt[1024];
    const bool second = (int)blockIdx.x >= a.blocks;
    const OrderJob j = second ? b : a;
    const int i = (second ? blockIdx.x - a.blocks : blockIdx.x) * blockDim.x + threadIdx.x;
    const int n = j.n;
    if (n > 65536) {
        if (i < n) j.order[i] = i;
        return;
    }
    const int ci = i < n ? j.ptr[i + 1] - j.ptr[i] : 0;
    int rank = 0;
    for (int j0 = 0; j0 < n; j0 += 1024) {
        __syncthreads();
        for (int c = threadIdx.x; c < 1024; c += blockDim.x)
            cnt[c] = (j0 + c < n) ? j.ptr[j0 + c + 1] - j.ptr[j0 + c] : -1;
        __syncthreads();
        const int jn = min(1024, n - j0);
#pragma unroll 8
        for (int c = 0; c < jn; ++c) {
            const int cj = cnt[c];
            rank += (cj > ci) || (cj == ci && j0 + c < i);
        }
    }
    if (i < n) j.order[rank] = i;
}

static ListJob list_job(const uint8_t* src, const ListGeom& g, int* ptr, int* ent, int tag_full) {
    return ListJob{src, g, ptr, ent, tag_full, (g.nlists + 3) / 4};
}

static hipError_t run_lists(const ListJob& a, const ListJob& b, hipStream_t s) {
    const unsigned blocks = (unsigned)(a.blocks + b.blocks);
    hipLaunchKernelGGL(list_count_kernel, dim3(blocks), dim3(256), 0, s, a, b);
    hipLaunchKernelGGL(scan_kernel, dim3(2), dim3(1024), 0, s, a, b);
    hipLaunchKernelGGL(list_fill_kernel, dim3(blocks), dim3(256), 0, s, a, b);
    return hipGetLastError();
}

int launch_index_dense(const Problem& P, const int32_t* desc_words, void* index, void* stream) {
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const int4* desc = reinterpret_cast<const int4*>(desc_words);
    const IndexLayout L = index_layout(P);
    char* base = static_cast<char*>(index);
    uint8_t* fcls = reinterpret_cast<uint8_t*>(base + L.fwd_cls);
    uint8_t* bcls = reinterpret_cast<uint8_t*>(base + L.bwd_cls);
    int* fptr = reinterpret_cast<int*>(base + L.fwd_ptr);
    int* fent = reinterpret_cast<int*>(base + L.fwd_ent);
    int* ford = reinterpret_cast<int*>(base + L.fwd_order);
    int* bptr = reinterpret_cast<int*>(base + L.bwd_ptr);
    int* bent = reinterpret_cast<int*>(base + L.bwd_ent);
    int* bord = reinterpret_cast<int*>(base + L.bwd_order);

    const long nf = (long)P.nqt_f * P.nkt_f, nbk = (long)P.nqt_b * P.nkt_b;
    const ClassifyJob cf{P.fBM, P.fBN, P.nqt_f, P.nkt_f, fcls, (int)((nf + 255) / 256)};
    const ClassifyJob cb{P.bBM, P.bBN, P.nqt_b, P.nkt_b, bcls, (int)((nbk + 255) / 256)};
    hipLaunchKernelGGL(classify_kernel, dim3((unsigned)(cf.blocks + cb.blocks)), dim3(256), 0, s, desc, P.T, cf, cb);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
    // forward: rows of the class map (one list per query tile); backward: its columns (one
    // list per key tile)
    const ListJob lf = list_job(fcls, ListGeom{P.nqt_f, P.nkt_f, 1, P.nkt_f, 0, 1}, fptr, fent, 1);
    const ListJob lb = list_job(bcls, ListGeom{P.nkt_b, P.nqt_b, 1, 1, 0, P.nkt_b}, bptr, bent, 1);
    if ((e = run_lists(lf, lb, s)) != hipSuccess) return (int)e;
    const OrderJob of{fptr, P.nqt_f, ford, (P.nqt_f + 255) / 256};
    const OrderJob ob{bptr, P.nkt_b, bord, (P.nkt_b + 255) / 256};
    hipLaunchKernelGGL(order_kernel, dim3((unsigned)(of.blocks + ob.blocks)), dim3(256), 0, s, of, ob);
    return (int)hipGetLastError();
}

int launch_index_sparse(const Problem& P, const uint8_t* keep, void* index, void* stream) {
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const IndexLayout L = index_layout(P);
    char* base = static_cast<char*>(index);
    int* fptr = reinterpret_cast<int*>(base + L.fwd_ptr);
    int* fent = reinterpret_cast<int*>(base + L.fwd_ent);
    int* bptr = reinterpret_cast<int*>(base + L.bwd_ptr);
    int* bent = reinterpret_cast<int*>(base + L.bwd_ent);
    const int nb = P.nb;
    // rows (h, qb): keep[(h * nb + qb) * nb + kb], entries kb;
    // columns (g, kb): elements m = hi * nb + qb at keep[((g*G + hi) * nb + qb) * nb + kb]
    const ListJob lf = list_job(keep, ListGeom{P.Hq * nb, nb, 1, nb, 0, 1}, fptr, fent, 0);
    const ListJob lb = list_job(keep, ListGeom{P.Hk * nb, P.G * nb, nb, (long)P.G * nb * nb, 1, nb}, bptr, bent, 0);
    return (int)run_lists(lf, lb, s);
}

}  // namespace mlct
