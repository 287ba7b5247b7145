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

// One thread per tile. Threads of a wave share the key tile (consecutive query tiles),
// so the descriptor reads are broadcast.
__global__ void classify_kernel(const int4* __restrict__ desc, int T, int BM, int BN, int nqt, int nkt,
                                uint8_t* __restrict__ cls) {
    const long t = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= (long)nqt * nkt) return;
    const int kt = (int)(t / nqt), qt = (int)(t % nqt);
    const int r0 = qt * BM, r1 = min(T, r0 + BM);
    const int c0 = kt * BN, c1 = min(T, c0 + BN);
    const int rows = r1 - r0;
    bool any = false, all = true;
    for (int j = c0; j < c1; ++j) {
        const int4 d = desc[j];
        const int n0 = max(0, min(d.y, r1) - max(d.x, r0));
        const int n1 = max(0, min(d.w, r1) - max(d.z, r0));
        const int n = n0 + n1;
        any |= n > 0;
        all &= n == rows;
    }
    cls[(size_t)qt * nkt + kt] = any ? (all ? CLS_FULL : CLS_PARTIAL) : CLS_EMPTY;
}

// Lists: list l has `len` elements; element m of list l is at
//   src[(l / div) * s_hi + (l % div) * s_lo + m * s_m].
struct ListGeom {
    int nlists, len, div;
    long s_hi, s_lo, s_m;
};

__device__ __forceinline__ size_t elem_addr(const ListGeom& g, int l, int m) {
    return (size_t)((long)(l / g.div) * g.s_hi + (long)(l % g.div) * g.s_lo + (long)m * g.s_m);
}

// One wave per list: count non-zero elements into ptr[l + 1] (ptr[0] = 0).
__global__ void list_count_kernel(const uint8_t* __restrict__ src, ListGeom g, int* __restrict__ ptr) {
    const int wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int lane = threadIdx.x & 63;
    if (wave >= g.nlists) return;
    int count = 0;
    for (int m0 = 0; m0 < g.len; m0 += 64) {
        const int m = m0 + lane;
        const bool nz = m < g.len && src[elem_addr(g, wave, m)] != 0;
        count += __popcll(__ballot(nz));
    }
    if (lane == 0) {
        ptr[wave + 1] = count;
        if (wave == 0) ptr[0] = 0;
    }
}

// One wave per list: write the indices of non-zero elements in ascending order,
// (m << 1) | (value == FULL) when tag_full, else m.
__global__ void list_fill_kernel(const uint8_t* __restrict__ src, ListGeom g, const int* __restrict__ ptr,
                                 int* __restrict__ ent, int tag_full) {
    const int wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int lane = threadIdx.x & 63;
    if (wave >= g.nlists) return;
    int base = ptr[wave];
    const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int m0 = 0; m0 < g.len; m0 += 64) {
        const int m = m0 + lane;
        const uint8_t v = m < g.len ? src[elem_addr(g, wave, m)] : 0;
        const unsigned long long b = __ballot(v != 0);
        if (v != 0) ent[base + __popcll(b & below)] = tag_full ? ((m << 1) | (v == CLS_FULL)) : m;
        base += __popcll(b);
    }
}

// In-place inclusive prefix sum of a[1..n] (a[0] = 0), one workgroup of 1024 threads.
__global__ __launch_bounds__(1024) void scan_kernel(int* __restrict__ a, int n) {
    __shared__ int part[1024];
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

// order[rank] = i, ranks by descending list length, ties by ascending index.
__global__ void order_kernel(const int* __restrict__ ptr, int n, int* __restrict__ order) {
    __shared__ int cnt[1024];
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    const int ci = i < n ? ptr[i + 1] - ptr[i] : 0;
    int rank = 0;
    for (int j0 = 0; j0 < n; j0 += 1024) {
        __syncthreads();
        for (int j = threadIdx.x; j < 1024; j += blockDim.x)
            cnt[j] = (j0 + j < n) ? ptr[j0 + j + 1] - ptr[j0 + j] : -1;
        __syncthreads();
        const int jn = min(1024, n - j0);
        for (int j = 0; j < jn; ++j) {
            const int cj = cnt[j];
            rank += (cj > ci) || (cj == ci && j0 + j < i);
        }
    }
    if (i < n) order[rank] = i;
}

__global__ void identity_kernel(int* __restrict__ order, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) order[i] = i;
}

static hipError_t run_lists(const uint8_t* src, const ListGeom& g, int* ptr, int* ent, int tag_full,
                            hipStream_t s) {
    const int waves_per_block = 4;
    const int blocks = (g.nlists + waves_per_block - 1) / waves_per_block;
    hipLaunchKernelGGL(list_count_kernel, dim3(blocks), dim3(64 * waves_per_block), 0, s, src, g, ptr);
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, s, ptr, g.nlists);
    hipLaunchKernelGGL(list_fill_kernel, dim3(blocks), dim3(64 * waves_per_block), 0, s, src, g, ptr, ent,
                       tag_full);
    return hipGetLastError();
}

static hipError_t run_order(const int* ptr, int n, int* order, hipStream_t s) {
    const int blocks = (n + 255) / 256;
    if (n <= 65536)
        hipLaunchKernelGGL(order_kernel, dim3(blocks), dim3(256), 0, s, ptr, n, order);
    else
        hipLaunchKernelGGL(identity_kernel, dim3(blocks), dim3(256), 0, s, order, n);
    return hipGetLastError();
}

hipError_t launch_index_dense(const Problem& P, const int4* desc, void* index, hipStream_t s) {
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
    hipLaunchKernelGGL(classify_kernel, dim3((unsigned)((nf + 255) / 256)), dim3(256), 0, s, desc, P.T, P.fBM,
                       P.fBN, P.nqt_f, P.nkt_f, fcls);
    hipLaunchKernelGGL(classify_kernel, dim3((unsigned)((nbk + 255) / 256)), dim3(256), 0, s, desc, P.T, P.bBM,
                       P.bBN, P.nqt_b, P.nkt_b, bcls);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // forward: rows of the class map (one list per query tile)
    ListGeom gf{P.nqt_f, P.nkt_f, 1, P.nkt_f, 0, 1};
    if ((e = run_lists(fcls, gf, fptr, fent, 1, s)) != hipSuccess) return e;
    // backward: columns of the class map (one list per key tile)
    ListGeom gb{P.nkt_b, P.nqt_b, 1, 1, 0, P.nkt_b};
    if ((e = run_lists(bcls, gb, bptr, bent, 1, s)) != hipSuccess) return e;
    if ((e = run_order(fptr, P.nqt_f, ford, s)) != hipSuccess) return e;
    return run_order(bptr, P.nkt_b, bord, s);
}

hipError_t launch_index_sparse(const Problem& P, const uint8_t* keep, void* index, hipStream_t s) {
    const IndexLayout L = index_layout(P);
    char* base = static_cast<char*>(index);
    int* fptr = reinterpret_cast<int*>(base + L.fwd_ptr);
    int* fent = reinterpret_cast<int*>(base + L.fwd_ent);
    int* bptr = reinterpret_cast<int*>(base + L.bwd_ptr);
    int* bent = reinterpret_cast<int*>(base + L.bwd_ent);
    const int nb = P.nb;
    // rows (h, qb): keep[(h * nb + qb) * nb + kb], entries kb
    ListGeom gf{P.Hq * nb, nb, 1, nb, 0, 1};
    hipError_t e = run_lists(keep, gf, fptr, fent, 0, s);
    if (e != hipSuccess) return e;
    // columns (g, kb): elements m = hi * nb + qb at keep[((g*G + hi) * nb + qb) * nb + kb]
    ListGeom gb{P.Hk * nb, P.G * nb, nb, (long)P.G * nb * nb, 1, nb};
    return run_lists(keep, gb, bptr, bent, 0, s);
}

}  // namespace mlct
