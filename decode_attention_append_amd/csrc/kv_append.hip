// KV append: the new K/V rows of a decode step are copied into the
// pre-allocated cache as one contiguous slice per (sequence, KV head),
// starting at that sequence's seq_pos ("Qwen MoE BringUp", Per-Layer IR
// Patterns, "KV Cache Update (EP rewrite: tensor.insert_slice)"; fix A5).
//
// One lane moves 16 bytes of K and 16 bytes of V: sixteen lanes cover one
// 128-dim row (32 a 256-dim row), a wave covers four (two) rows with fully
// coalesced 128-bit loads and stores.  Without a rotary table it is a pure bit copy: no arithmetic touches
// the data.  With one, each K row is rotated at its position seq_pos + i first
// (the RoPE block of the same page; lanes c and c ^ 8 of a row hold the two
// halves of each rotated pair and swap them with one shuffle).  In a paged
// cache the row's slot comes from the block table.
#include "da_internal.h"

namespace da {

template <bool F16>
__global__ __launch_bounds__(256) void kv_append_kernel(AppendParams p, int threads_total) {
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    const int lpr = p.head_dim / 8;   // lanes per row: 16 (head_dim 128) or 32 (256)
    const int piece = t % lpr;        // 16-byte piece of the row
    const int row = t / lpr;          // (b, i, h) in k_new's [B][q_len][Hkv] order
    const int h = row % p.n_kv_heads;
    const int i = (row / p.n_kv_heads) % p.q_len;
    const int b = min(row / (p.n_kv_heads * p.q_len), p.batch - 1);
    const int sp = p.seq_pos[b];
    // a sequence that breaks the contract is skipped (both lanes of every pair
    // belong to the same row, so they agree)
    const bool ok = t < threads_total && sp >= 0 && sp <= p.max_seq - p.q_len &&
                    kv_row_writable(p.layout, b, sp + i);
    const size_t src = (size_t)min(row, threads_total / lpr - 1) * (p.head_dim * 2) + piece * 16;
    u32x4_t k = ld16(p.k_new + src);
    if (p.rope_freqs) rope_row<F16>(k, piece, p.rope_dim, sp + i, p.rope_freqs, ok);
    if (!ok) return;
    const size_t dst = kv_row_off(p.layout, b, h, p.n_kv_heads, p.max_seq, sp + i) + piece * 16;
    const u32x4_t v = ld16(p.v_new + src);
    *reinterpret_cast<u32x4_t *>(p.k_cache + dst) = k;
    *reinterpret_cast<u32x4_t *>(p.v_cache + dst) = v;
}

hipError_t launch_kv_append(const AppendParams &p, int threads_total, bool fp16, hipStream_t s) {
    const int block = 256;
    const int grid = (threads_total + block - 1) / block;
    if (fp16)
        hipLaunchKernelGGL(kv_append_kernel<true>, dim3(grid), dim3(block), 0, s, p, threads_total);
    else
        hipLaunchKernelGGL(kv_append_kernel<false>, dim3(grid), dim3(block), 0, s, p, threads_total);
    return hipGetLastError();
}

// Zero fill of a small int32 array (the arrival counters of the one-launch
// step).  A kernel rather than a memset so that the call can be captured into
// a HIP graph.
__global__ __launch_bounds__(256) void fill_zero_kernel(int32_t *x, int n) {
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t < n) x[t] = 0;
}

hipError_t launch_fill_zero(int32_t *x, int n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((n + 255) / 256), dim3(256), 0, s, x, n);
    return hipGetLastError();
}

}  // namespace da
