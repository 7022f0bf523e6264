// kv_compact.hip -- commit the accepted path's K/V into contiguous cache slots.
//
// "Recurrent Drafter for Fast Speculative Decoding in Large Language Models",
// section "The Full Speculative Decoding Loop", Step 6: the accepted tokens are
// appended to the context and the next step starts after them.  The tree's K/V
// sit at slots ctx + node; the accepted path's entries move to ctx + 1.., the
// root staying at ctx.  A destination can be another entry's source
// (path [0, 2, 3]: slot ctx+2 is both), so a workgroup first gathers all the
// moved rows of its heads into LDS, then scatters them.
#include <algorithm>

#include "common.hpp"

namespace spec {
namespace {

constexpr int kThreads = 256;
constexpr int kBatch = 4;                     // 16-byte loads in flight per thread
constexpr long kBufWords = 64 * 1024 / 16;    // LDS buffer of a workgroup: 64 KiB

// One workgroup per (sequence, K or V, group of HPG KV heads), sized on the
// host so that the longest possible path of a group fits its LDS buffer; about
// 64 groups overall, so a small batch still spreads its rows over many CUs.
// Every workgroup of a sequence reads the context length, then adds one to the
// sequence's arrival counter in the workspace (after the read has returned);
// the workgroup that arrives last has seen every other arrival, so every other
// workgroup has read the old length by then: it writes the new length and
// returns the counter to zero for the next call.  ctx_len holds nothing but
// the length at any time.
__global__ __launch_bounds__(kThreads) void k_kv_compact(
    int elem_bytes, int Hkv, int HPG, int G, int D, int cache_cap, int T_cap,
    unsigned char* __restrict__ kc, unsigned char* __restrict__ vc, int32_t* __restrict__ ctx_len,
    const int32_t* __restrict__ acc_len, const int32_t* __restrict__ acc_path,
    uint32_t* __restrict__ arrivals, int32_t* __restrict__ status) {
  static_assert(kThreads >= SPEC_MAX_TREE, "one path entry per thread");
  extern __shared__ uint4 buf[];  // [HPG * longest path * row words]
  __shared__ int s_src[SPEC_MAX_TREE];
  __shared__ int s_ok, s_ctx, s_last;
  const int b = blockIdx.x;
  const int which = blockIdx.y / G;
  const int g = blockIdx.y - which * G;
  const int tid = threadIdx.x;
  // the length, the accepted count and the whole path row in one round trip;
  // entries past the accepted length are ignored
  const int n = acc_len[b];
  const int32_t* path = acc_path + (size_t)b * T_cap;
  const int my_src = tid < T_cap ? path[tid] : 0;
  if (tid == 0) {
    const int ctx = __hip_atomic_load(ctx_len + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // the length has arrived before the arrival is counted
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    const uint32_t before = __hip_atomic_fetch_add(arrivals + b, 1u, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
    s_ctx = ctx;
    s_last = before == (uint32_t)(2 * G - 1);
    s_ok = (n >= 0 && n < T_cap && ctx >= 0 && ctx + n + 1 <= cache_cap) ? 1 : 0;
  }
  if (tid < T_cap) s_src[tid] = my_src;
  __syncthreads();
  const int ctx = s_ctx;
  if (s_ok && tid >= 1 && tid <= n) {
    // node ids along a path increase strictly and are at least their depth
    if (my_src < tid || ctx + my_src >= cache_cap || (tid > 1 && my_src <= s_src[tid - 1]))
      atomicAnd(&s_ok, 0);
  }
  __syncthreads();
  if (s_ok) {
    const int row16 = D * elem_bytes / 16;  // 16-byte words per row
    const int per_head = n * row16;
    const int h0 = g * HPG;
    const int nh = min(HPG, Hkv - h0);
    const int total = nh * per_head;  // fits the LDS buffer (sized on the host)
    const size_t head_bytes = (size_t)cache_cap * D * elem_bytes;
    unsigned char* base = (which ? vc : kc) + ((size_t)b * Hkv + h0) * head_bytes;
    // kBatch loads in flight per thread: every load is issued (a unit past the
    // end reads the group's first word as a stand-in) and only the LDS store
    // is predicated, so the loads do not wait on one another
    auto unit = [&](int e, bool& keep) -> uint4 {
      const bool in = e < total;
      const int ec = in ? e : 0;
      const int h = ec / per_head, rem = ec - (ec / per_head) * per_head;
      const int i = 1 + rem / row16, w = rem - (rem / row16) * row16;
      const int src = s_src[i];
      keep = in && src != i;
      const size_t off = in ? h * head_bytes + (size_t)(ctx + src) * D * elem_bytes + w * 16 : 0;
      return *reinterpret_cast<const uint4*>(base + off);
    };
    for (int e0 = tid; e0 < total; e0 += kBatch * kThreads) {
      uint4 t[kBatch];
      bool keep[kBatch];
#pragma unroll
      for (int k = 0; k < kBatch; ++k) t[k] = unit(e0 + k * kThreads, keep[k]);
      __builtin_amdgcn_sched_barrier(0);  // keep the batch's loads ahead of its stores
#pragma unroll
      for (int k = 0; k < kBatch; ++k)
        if (keep[k]) buf[e0 + k * kThreads] = t[k];
    }
    __syncthreads();  // every source read before any destination is written
    for (int e = tid; e < total; e += kThreads) {
      const int h = e / per_head, rem = e - (e / per_head) * per_head;
      const int i = 1 + rem / row16, w = rem - (rem / row16) * row16;
      if (s_src[i] != i)
        reinterpret_cast<uint4*>(base + h * head_bytes + (size_t)(ctx + i) * D * elem_bytes)[w] =
            buf[e];
    }
  }
  if (tid == 0 && s_last) {
    // every other workgroup of the sequence has read the old length already
    ctx_len[b] = s_ok ? ctx + n + 1 : ctx;
    __hip_atomic_store(arrivals + b, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (!s_ok) raise_status(status, SPEC_DEV_CTX_RANGE);
  }
}

// Plain streaming copy, 16 bytes per thread per step, grid-stride.
__global__ __launch_bounds__(256) void k_copy_probe(const uint4* __restrict__ src,
                                                    uint4* __restrict__ dst, size_t n16) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    dst[i] = src[i];
}

// Plain streaming read for the achievable read rate: workgroup g reads the
// 256 KiB chunks g, g + grid, ... front to back, each thread two batches of
// four non-temporal 16-byte loads in flight (buffer loads, so the tail of a
// partial last chunk reads zeros).  One contiguous stream per workgroup and
// about four workgroups per CU is the fastest plain read measured on MI355X.
constexpr unsigned kProbeChunk = 256u << 10;

__global__ __launch_bounds__(256) void k_read_probe(const unsigned char* __restrict__ src,
                                                    size_t n_bytes, float* __restrict__ out) {
  constexpr int kU = 4;
  constexpr unsigned kPer = kProbeChunk / 16 / 256;  // 16-byte loads per thread per chunk
  static_assert(kPer % (2 * kU) == 0, "whole batches per chunk");
  const int tid = threadIdx.x;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const size_t n_chunks = (n_bytes + kProbeChunk - 1) / kProbeChunk;
  for (size_t c = blockIdx.x; c < n_chunks; c += gridDim.x) {
    const size_t left = n_bytes - c * kProbeChunk;
    const unsigned range = left < kProbeChunk ? (unsigned)left : kProbeChunk;
    const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(src + c * kProbeChunk),
                                                      (short)0, range, 0x00020000);
    f32x4 a[kU], b[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u)
      a[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (u * 256 + tid) * 16, 0, kLoadOnce));
    for (unsigned j0 = 0; j0 < kPer; j0 += 2 * kU) {
#pragma unroll
      for (int u = 0; u < kU; ++u)
        b[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                             rs, ((j0 + kU + u) * 256 + tid) * 16, 0, kLoadOnce));
#pragma unroll
      for (int u = 0; u < kU; ++u) acc += a[u];
      if (j0 + 2 * kU < kPer) {
#pragma unroll
        for (int u = 0; u < kU; ++u)
          a[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                               rs, ((j0 + 2 * kU + u) * 256 + tid) * 16, 0, kLoadOnce));
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) acc += b[u];
    }
  }
  __shared__ float s_sum[4];
  const float t = wave_sum_f32(acc[0] + acc[1] + acc[2] + acc[3]);
  if ((tid & 63) == 0) s_sum[tid >> 6] = t;
  __syncthreads();
  if (tid == 0) out[blockIdx.x] = s_sum[0] + s_sum[1] + s_sum[2] + s_sum[3];
}

}  // namespace
}  // namespace spec

using namespace spec;

extern "C" size_t spec_kv_compact_workspace_size(int B) {
  return B < 1 ? 0 : round_up((size_t)B * sizeof(uint32_t), 256);
}

extern "C" int spec_kv_compact(int dt, int B, int Hkv, int D, int cache_cap, int T_cap,
                               void* k_cache, void* v_cache, int32_t* ctx_len,
                               const int32_t* acc_len, const int32_t* acc_path, void* ws,
                               size_t ws_bytes, int32_t* status, void* stream) {
  if (B < 0 || Hkv < 1 || D < 1 || cache_cap < 1 || T_cap < 1) return SPEC_ERR_INVALID;
  if (T_cap > SPEC_MAX_TREE) return SPEC_ERR_CAPACITY;
  const int eb = dt == SPEC_F32 ? 4 : dt == SPEC_BF16 ? 2 : 0;
  if (!eb) return SPEC_ERR_INVALID;
  if ((D * eb) % 16) return SPEC_ERR_UNSUPPORTED;
  // heads per workgroup: the longest path a group can commit fits 64 KiB of LDS
  const long per_head_max = (long)(T_cap - 1 > 0 ? T_cap - 1 : 1) * D * eb / 16;
  if (per_head_max > kBufWords) return SPEC_ERR_UNSUPPORTED;
  if (B == 0) return SPEC_OK;
  if (!k_cache || !v_cache || !ctx_len || !acc_len || !acc_path) return SPEC_ERR_INVALID;
  if (!aligned(k_cache, 16) || !aligned(v_cache, 16)) return SPEC_ERR_INVALID;
  if (!ws || ws_bytes < spec_kv_compact_workspace_size(B) || !aligned(ws, 256))
    return SPEC_ERR_WORKSPACE;
  int HPG = (int)(kBufWords / per_head_max);
  if (HPG > Hkv) HPG = Hkv;
  // small batches get more groups (more workgroups in flight), large ones
  // fewer (fewer same-address arrivals per sequence): about 64 groups overall
  const int g_min = (Hkv + HPG - 1) / HPG;  // fewest groups the buffer allows
  const int g_want = std::min(Hkv, (64 + B - 1) / B);
  if (g_want > g_min) HPG = (Hkv + g_want - 1) / g_want;
  const int G = (Hkv + HPG - 1) / HPG;
  const size_t lds = (size_t)HPG * per_head_max * 16;
  status = status_or_library(status);
  hipLaunchKernelGGL(k_kv_compact, dim3(B, 2 * G), dim3(kThreads), lds, as_stream(stream), eb,
                     Hkv, HPG, G, D, cache_cap, T_cap, static_cast<unsigned char*>(k_cache),
                     static_cast<unsigned char*>(v_cache), ctx_len, acc_len, acc_path,
                     static_cast<uint32_t*>(ws), status);
  return launch_status();
}

extern "C" int spec_copy_probe(const void* src, void* dst, size_t n_bytes, void* stream) {
  if (!src || !dst || n_bytes % 16 || !aligned(src, 16) || !aligned(dst, 16))
    return SPEC_ERR_INVALID;
  if (n_bytes == 0) return SPEC_OK;
  const size_t n16 = n_bytes / 16;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(k_copy_probe, dim3((unsigned)blocks), dim3(256), 0, as_stream(stream),
                     static_cast<const uint4*>(src), static_cast<uint4*>(dst), n16);
  return launch_status();
}

extern "C" int spec_read_probe(const void* src, size_t n_bytes, float* out, int n_blocks,
                               void* stream) {
  if (!src || !out || n_bytes % 16 || !aligned(src, 16) || n_blocks < 1) return SPEC_ERR_INVALID;
  if (n_bytes == 0) return SPEC_OK;
  hipLaunchKernelGGL(k_read_probe, dim3((unsigned)n_blocks), dim3(256), 0, as_stream(stream),
                     static_cast<const unsigned char*>(src), n_bytes, out);
  return launch_status();
}

extern "C" int spec_version(void) { return 100; }

extern "C" const char* spec_status_string(int status) {
  switch (status) {
    case SPEC_OK: return "SPEC_OK";
    case SPEC_ERR_INVALID: return "SPEC_ERR_INVALID";
    case SPEC_ERR_UNSUPPORTED: return "SPEC_ERR_UNSUPPORTED";
    case SPEC_ERR_CAPACITY: return "SPEC_ERR_CAPACITY";
    case SPEC_ERR_WORKSPACE: return "SPEC_ERR_WORKSPACE";
    case SPEC_ERR_HIP: return "SPEC_ERR_HIP";
    default: return "SPEC_ERR_UNKNOWN";
  }
}
