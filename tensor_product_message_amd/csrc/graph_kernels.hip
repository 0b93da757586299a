// Graph bookkeeping on the device: the sender-sorted transpose of a
// CSR-by-receiver graph and a graph checker.
//
// The backward pass gathers each sender's out-edges in CSR edge order
// (FlashCart, arXiv 2610.06409: edges ordered by sender make sender-gradient
// accumulation deterministic).  The transpose is built without scratch memory:
//   1. count out-degrees into send_ptr[s + 2] (integer atomics: exact);
//   2. inclusive scan of send_ptr[0..N], so send_ptr[s + 1] = first slot of s;
//   3. place every edge with an atomic cursor on send_ptr[s + 1], which leaves
//      send_ptr[s + 1] = one past the last slot of s, i.e. the final pointers;
//   4. sort each sender's segment ascending (restores CSR order exactly; a
//      bitonic network per sender, one workgroup each);
//   5. send_recv[k] = receiver of send_perm[k] by binary search in row_ptr.
// Integer atomics make steps 1-3 order-independent in result after step 4, so
// the output is bit-exact and identical from run to run.
#include <hip/hip_runtime.h>

#include "kernels.hpp"

namespace ctp {

namespace {

__global__ void k_fill_i32(int32_t* __restrict__ p, long n, int32_t v) {
    long k = (long)blockIdx.x * blockDim.x + threadIdx.x;
    const long stride = (long)gridDim.x * blockDim.x;
    for (; k < n; k += stride) p[k] = v;
}

__global__ void k_count(int n_nodes, int n_edges, const int32_t* __restrict__ senders, int32_t* send_ptr) {
    long e = (long)blockIdx.x * blockDim.x + threadIdx.x;
    const long stride = (long)gridDim.x * blockDim.x;
    for (; e < n_edges; e += stride) {
        const int s = senders[e];
        if (s >= 0 && s + 2 <= n_nodes) atomicAdd(send_ptr + s + 2, 1);
    }
}

// Inclusive scan of a[0..n) in one workgroup of 1024 threads, chunk by chunk.
__global__ void __launch_bounds__(1024) k_scan_inclusive(int32_t* a, long n) {
    __shared__ int32_t part[1024];
    __shared__ int32_t carry;
    const int t = threadIdx.x;
    if (t == 0) carry = 0;
    __syncthreads();
    for (long base = 0; base < n; base += 1024) {
        const long k = base + t;
        int32_t v = k < n ? a[k] : 0;
        part[t] = v;
        __syncthreads();
        for (int off = 1; off < 1024; off <<= 1) {
            const int32_t add = t >= off ? part[t - off] : 0;
            __syncthreads();
            part[t] += add;
            __syncthreads();
        }
        if (k < n) a[k] = part[t] + carry;
        __syncthreads();
        if (t == 1023) carry += part[1023];
        __syncthreads();
    }
}

__global__ void k_place(int n_nodes, int n_edges, const int32_t* __restrict__ senders, int32_t* send_ptr,
                        int32_t* __restrict__ send_perm) {
    long e = (long)blockIdx.x * blockDim.x + threadIdx.x;
    const long stride = (long)gridDim.x * blockDim.x;
    for (; e < n_edges; e += stride) {
        const int s = senders[e];
        if (s < 0 || s >= n_nodes) continue;    // invalid graph: result undefined, but no stray write
        const int slot = atomicAdd(send_ptr + s + 1, 1);
        send_perm[slot] = static_cast<int32_t>(e);
    }
}

// One workgroup per sender sorts its segment ascending (the keys are
// distinct edge ids, so the sorted order is unique) with a bitonic network:
// O(n log^2 n) work, O(log^2 n) barrier-separated stages.  Segments up to
// kSortLds elements are sorted in LDS, padded to a power of two with INT_MAX;
// longer ones (hubs) in place in global memory, where every comparator puts
// the smaller key at the lower index and comparators that reach past the
// segment's end are skipped (the missing elements act as +infinity and would
// stay in place), so no padding is needed.
constexpr int kSortThreads = 256;
constexpr int kSortLds = 4096;

__device__ __forceinline__ void cmp_swap(int32_t* a, int i, int j) {
    const int32_t x = a[i], y = a[j];
    if (y < x) {
        a[i] = y;
        a[j] = x;
    }
}

// Bitonic sort of a[0..n) (n <= m, m a power of two) by the "flip" network:
// in merge stage k the first comparator of each block of size k pairs i with
// its mirror image, the later ones pair i with i + j.
__device__ void bitonic_sort(int32_t* a, int n, int m, int tid, int nth) {
    for (int k = 2; k <= m; k <<= 1) {
        for (int t = tid; t < m / 2; t += nth) {
            const int blk = t / (k / 2), off = t % (k / 2);
            const int i = blk * k + off, j = blk * k + k - 1 - off;
            if (j < n) cmp_swap(a, i, j);
        }
        __syncthreads();
        for (int j2 = k / 4; j2 >= 1; j2 >>= 1) {
            for (int t = tid; t < m / 2; t += nth) {
                const int blk = t / j2, off = t % j2;
                const int i = blk * 2 * j2 + off, j = i + j2;
                if (j < n) cmp_swap(a, i, j);
            }
            __syncthreads();
        }
    }
}

__global__ void __launch_bounds__(kSortThreads)
k_sort_segments(const int32_t* __restrict__ send_ptr, int32_t* __restrict__ send_perm) {
    __shared__ int32_t buf[kSortLds];
    const int s = blockIdx.x, tid = threadIdx.x;
    const int b = send_ptr[s], n = send_ptr[s + 1] - b;
    if (n < 2) return;
    int m = 2;
    while (m < n) m <<= 1;
    if (m <= kSortLds) {
        for (int t = tid; t < m; t += kSortThreads) buf[t] = t < n ? send_perm[b + t] : 0x7fffffff;
        __syncthreads();
        bitonic_sort(buf, m, m, tid, kSortThreads);
        for (int t = tid; t < n; t += kSortThreads) send_perm[b + t] = buf[t];
    } else {
        // the workgroup's writes to global memory are visible to it after each barrier
        bitonic_sort(send_perm + b, n, m, tid, kSortThreads);
    }
}

__global__ void k_recv_of(int n_nodes, int n_edges, const int32_t* __restrict__ row_ptr,
                          const int32_t* __restrict__ send_perm, int32_t* __restrict__ send_recv) {
    long k = (long)blockIdx.x * blockDim.x + threadIdx.x;
    const long stride = (long)gridDim.x * blockDim.x;
    for (; k < n_edges; k += stride) {
        const int e = send_perm[k];
        int lo = 0, hi = n_nodes;       // last i with row_ptr[i] <= e
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (row_ptr[mid] <= e) lo = mid; else hi = mid;
        }
        send_recv[k] = lo;
    }
}

__global__ void k_check(int n_nodes, int n_edges, const int32_t* __restrict__ row_ptr,
                        const int32_t* __restrict__ senders, unsigned long long* bad) {
    long k = (long)blockIdx.x * blockDim.x + threadIdx.x;
    const long stride = (long)gridDim.x * blockDim.x;
    unsigned long long local = 0;
    for (long q = k; q < n_nodes; q += stride) local += row_ptr[q + 1] < row_ptr[q];
    for (long q = k; q < n_edges; q += stride) local += (senders[q] < 0) | (senders[q] >= n_nodes);
    if (k == 0) local += (row_ptr[0] != 0) + (row_ptr[n_nodes] != n_edges);
    if (local) atomicAdd(bad, local);
}

unsigned grid_for(long n, int block) {
    long g = (n + block - 1) / block;
    if (g < 1) g = 1;
    if (g > 65536) g = 65536;
    return static_cast<unsigned>(g);
}

}  // namespace

hipError_t launch_transpose(int n_nodes, int n_edges, const int32_t* row_ptr, const int32_t* senders,
                            int32_t* send_ptr, int32_t* send_perm, int32_t* send_recv, hipStream_t st) {
    const long np = (long)n_nodes + 1;
    hipLaunchKernelGGL(k_fill_i32, dim3(grid_for(np, 256)), dim3(256), 0, st, send_ptr, np, 0);
    if (n_edges > 0) {
        hipLaunchKernelGGL(k_count, dim3(grid_for(n_edges, 256)), dim3(256), 0, st, n_nodes, n_edges, senders,
                           send_ptr);
        hipLaunchKernelGGL(k_scan_inclusive, dim3(1), dim3(1024), 0, st, send_ptr, np);
        hipLaunchKernelGGL(k_place, dim3(grid_for(n_edges, 256)), dim3(256), 0, st, n_nodes, n_edges, senders,
                           send_ptr, send_perm);
        if (n_nodes > 0)
            hipLaunchKernelGGL(k_sort_segments, dim3(n_nodes), dim3(kSortThreads), 0, st, send_ptr, send_perm);
        hipLaunchKernelGGL(k_recv_of, dim3(grid_for(n_edges, 256)), dim3(256), 0, st, n_nodes, n_edges, row_ptr,
                           send_perm, send_recv);
    }
    return hipGetLastError();
}

hipError_t launch_check_graph(int n_nodes, int n_edges, const int32_t* row_ptr, const int32_t* senders,
                              unsigned long long* d_bad, hipStream_t st) {
    const long n = (long)(n_nodes > n_edges ? n_nodes : n_edges);
    hipLaunchKernelGGL(k_check, dim3(grid_for(n, 256)), dim3(256), 0, st, n_nodes, n_edges, row_ptr, senders, d_bad);
    return hipGetLastError();
}

}  // namespace ctp
