// ceilings.hip -- measured MI355X (gfx950) ceilings for the roofline figures of the
// SparseFlashAttentionGrad kernels: bf16 MFMA rate and the shader clock under MFMA load, HBM
// copy bandwidth, LDS instruction rates, the fp32 global atomic-add rate and the rate of the
// direct-to-LDS key-row gather in two lane mappings.  Not part of the
// library's C ABI; bench.py --ceilings loads it and prints the results.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// 8 independent accumulation chains of v_mfma_f32_16x16x32_bf16 per wave, `iters` rounds.  The
// MFMAs are written as inline asm with the accumulator tied to the destination so that each
// chain stays in place (no memory access in the asm).  Wave 0 of workgroup 0 records the
// shader-clock counter (s_memtime) and the 100 MHz constant counter (s_memrealtime) around its
// loop, so that clk[1] / clk[0] cycles per tick give the shader clock under MFMA load.
__global__ void __launch_bounds__(256) mfma_rate_kernel(float* out, int iters, unsigned long long* clk) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(0.001f * (lane + e));
    b[e] = (__bf16)(0.002f * (lane - e));
  }
  f32x4 c0{}, c1{}, c2{}, c3{}, c4{}, c5{}, c6{}, c7{};
  const bool timer = blockIdx.x == 0 && threadIdx.x == 0;
  unsigned long long t0 = 0, r0 = 0;
  if (timer) {
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
#define CEIL_MFMA(c) asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b))
  for (int it = 0; it < iters; ++it) {
    CEIL_MFMA(c0); CEIL_MFMA(c1); CEIL_MFMA(c2); CEIL_MFMA(c3);
    CEIL_MFMA(c4); CEIL_MFMA(c5); CEIL_MFMA(c6); CEIL_MFMA(c7);
  }
#undef CEIL_MFMA
  // results are read only after this wait-free dependency point; s_nop covers the last MFMAs
  asm volatile("s_nop 7\n s_nop 7\n s_nop 7" ::);
  const f32x4 sum = c0 + c1 + c2 + c3 + c4 + c5 + c6 + c7;
  const float s = sum[0] + sum[1] + sum[2] + sum[3];
  if (timer) {
    asm volatile("" ::"v"(s));
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    clk[0] = r1 - r0;
    clk[1] = t1 - t0;
  }
  if (s == 12345.f) out[blockIdx.x] = s;   // keeps the chains live; never true in practice
}

__global__ void __launch_bounds__(256) copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

// LDS instruction rate.  mode 0: ds_add_f32 (result unused), 1: ds_write_b32, 2: ds_read_b32,
// 3: ds_write_b128, 4: ds_read_b128, 5: ds_read_b64_tr_b16 (transposing read).  Each wave works
// on its own 16 KB region; in one round a lane issues 16 instructions at 16 distinct addresses
// (lanes of a wave address consecutive elements: conflict-free), every loaded element is
// consumed and every store survives (the round ends with a compiler barrier).
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;
__global__ void __launch_bounds__(256) lds_rate_kernel(int mode, int iters, float* out) {
  __shared__ __attribute__((aligned(16))) float buf[4 * 4096];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float* w = buf + wave * 4096;
  for (int i = lane; i < 4096; i += 64) w[i] = 0.f;
  __syncthreads();
  float acc = 0.f;
  int iacc = 0;
  for (int it = 0; it < iters; ++it) {
    const float v = 1.0f + lane + it;
    if (mode == 0) {
#pragma unroll
      for (int j = 0; j < 16; ++j) atomicAdd(&w[j * 256 + lane], v);
    } else if (mode == 1) {
#pragma unroll
      for (int j = 0; j < 16; ++j) w[j * 256 + lane] = v + j;
    } else if (mode == 2) {
#pragma unroll
      for (int j = 0; j < 16; ++j) acc += w[j * 256 + lane];
    } else if (mode == 3) {
#pragma unroll
      for (int j = 0; j < 16; ++j) reinterpret_cast<float4*>(w)[j * 64 + lane] = make_float4(v, v + j, v, v);
    } else if (mode == 4) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float4 x = reinterpret_cast<const float4*>(w)[j * 64 + lane];
        acc += (x.x + x.y) + (x.z + x.w);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const i16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4_t*)(reinterpret_cast<short*>(w) + j * 512 + 4 * lane));
        iacc += (x[0] ^ x[1]) + (x[2] ^ x[3]);
      }
    }
    asm volatile("" ::: "memory");
  }
  __syncthreads();
  acc += w[lane] + (float)iacc;
  if (acc == 12345.f) out[blockIdx.x] = acc;
}

// fp32 global atomic add (result unused): workgroup w adds 1.0 to every element of row
// rows[w] (1088 floats) `reps` times.  Rows repeat across workgroups as the index list says.
__global__ void __launch_bounds__(256) atomic_rate_kernel(float* acc, const int32_t* rows, int reps) {
  float* r = acc + (int64_t)rows[blockIdx.x] * 1088;
  for (int k = 0; k < reps; ++k)
    for (int e = threadIdx.x; e < 1088; e += 256) atomicAdd(&r[e], 1.0f);
}

// Direct-to-LDS gather of 32 key rows (a 1024-byte value row and a 128-byte rope row each) per
// chunk: the query-major kernels' key-tile fill.  Waves 4-7 of a 512-thread workgroup issue the
// 36 loads of 1 KB per chunk (9 each) into one of 4 LDS buffers, two chunks in flight; waves 0-3
// only pass the barriers.  mode 0: each load covers 32 bytes of 32 different keys (lane l: key
// l % 32, 16-byte piece 2 b + l / 32 of block b); mode 1: each load covers the whole 128-byte
// runs of 8 keys (lane l: key 8 q + l / 8, piece l % 8 of run g for load (g, q)).  idx holds nch
// chunks of 32 key numbers per workgroup, each below nkeys.
constexpr int kGatherChunkBytes = 36 * 1024;
__global__ void __launch_bounds__(512, 1) gather_rate_kernel(int mode, const char* kv, const char* kr,
                                                             const int32_t* idx, int nch, float* out) {
  __shared__ __attribute__((aligned(16))) char b0[kGatherChunkBytes], b1[kGatherChunkBytes],
      b2[kGatherChunkBytes], b3[kGatherChunkBytes];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int32_t* wg = idx + (size_t)blockIdx.x * nch * 32;
  const bool gw = wave >= 4;
  const int q = wave - 4;
  auto issue = [&](int ch) {
    if (!gw || ch >= nch) return;
    const int32_t* keys = wg + ch * 32;
    char* dst = (ch & 3) == 0 ? b0 : (ch & 3) == 1 ? b1 : (ch & 3) == 2 ? b2 : b3;
#pragma unroll
    for (int j = 0; j < 9; ++j) {
      const int i = q + 4 * j;                 // load index 0 .. 35 (32 .. 35: rope)
      int key, off;
      bool rope;
      if (mode == 0) {
        key = lane & 31;
        const int piece = 2 * i + (lane >> 5);
        rope = piece >= 64;
        off = (rope ? piece - 64 : piece) * 16;
      } else {
        rope = i >= 32;
        key = 8 * (i & 3) + (lane >> 3);
        off = ((rope ? 0 : (i >> 2) * 8) + (lane & 7)) * 16;
      }
      const int k = keys[key];
      const char* src = rope ? kr + (size_t)k * 128 + off : kv + (size_t)k * 1024 + off;
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(dst + i * 1024), 16, 0, 0);
    }
  };
  issue(0);
  issue(1);
  float acc = 0.f;
  for (int ch = 0; ch < nch; ++ch) {
    issue(ch + 2);
    // this wave's loads of chunk ch done: chunks ch + 1 and ch + 2 (18 loads) may remain
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((18 & 15) | ((18 >> 4) << 14) | (0x7 << 4));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    const char* rb = (ch & 3) == 0 ? b0 : (ch & 3) == 1 ? b1 : (ch & 3) == 2 ? b2 : b3;
    acc += (float)rb[threadIdx.x * 16];
  }
  if (acc == 12345.f) out[blockIdx.x] = acc;
}

extern "C" {

int ceil_device_info(char* name, int name_len, int* cus, int* clock_khz, int* mem_clock_khz) {
  hipDeviceProp_t p;
  if (hipGetDeviceProperties(&p, 0) != hipSuccess) return -1;
  // marketing name, then the architecture name (the former can be empty in containers)
  const char* src = p.name[0] ? p.name : p.gcnArchName;
  int i = 0;
  for (; i < name_len - 1 && src[i]; ++i) name[i] = src[i];
  if (p.name[0]) {
    const char* arch = p.gcnArchName;
    if (i + 2 < name_len - 1) {
      name[i++] = ' ';
      name[i++] = '(';
      for (; i < name_len - 2 && *arch; ++i) name[i] = *arch++;
      name[i++] = ')';
    }
  }
  name[i] = 0;
  *cus = p.multiProcessorCount;
  *clock_khz = p.clockRate;
  *mem_clock_khz = p.memoryClockRate;
  return 0;
}

// Each call runs one launch on `stream` and returns its elapsed ms from HIP events (-1: error).
static float timed(hipStream_t s, void (*launch)(hipStream_t, void*), void* ctx) {
  hipEvent_t a, b;
  if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) return -1.f;
  float ms = -1.f;
  if (hipEventRecord(a, s) == hipSuccess) {
    launch(s, ctx);
    if (hipGetLastError() == hipSuccess && hipEventRecord(b, s) == hipSuccess && hipEventSynchronize(b) == hipSuccess &&
        hipEventElapsedTime(&ms, a, b) != hipSuccess)
      ms = -1.f;
  }
  (void)hipEventDestroy(a);
  (void)hipEventDestroy(b);
  return ms;
}

struct MfmaCtx { float* out; int blocks, iters; unsigned long long* clk; };
static void mfma_launch(hipStream_t s, void* c) {
  MfmaCtx* x = (MfmaCtx*)c;
  hipLaunchKernelGGL(mfma_rate_kernel, dim3(x->blocks), dim3(256), 0, s, x->out, x->iters, x->clk);
}
float ceil_mfma(float* out, int blocks, int iters, unsigned long long* clk_dev, void* stream) {
  MfmaCtx c{out, blocks, iters, clk_dev};
  return timed((hipStream_t)stream, mfma_launch, &c);
}

struct CopyCtx { const void* src; void* dst; size_t n16; int blocks; };
static void copy_launch(hipStream_t s, void* c) {
  CopyCtx* x = (CopyCtx*)c;
  hipLaunchKernelGGL(copy_kernel, dim3(x->blocks), dim3(256), 0, s, (const uint4*)x->src, (uint4*)x->dst, x->n16);
}
float ceil_copy(const void* src, void* dst, size_t bytes, int blocks, void* stream) {
  CopyCtx c{src, dst, bytes / 16, blocks};
  return timed((hipStream_t)stream, copy_launch, &c);
}

struct LdsCtx { int mode, iters, blocks; float* out; };
static void lds_launch(hipStream_t s, void* c) {
  LdsCtx* x = (LdsCtx*)c;
  hipLaunchKernelGGL(lds_rate_kernel, dim3(x->blocks), dim3(256), 0, s, x->mode, x->iters, x->out);
}
float ceil_lds(int mode, int blocks, int iters, float* out, void* stream) {
  LdsCtx c{mode, iters, blocks, out};
  return timed((hipStream_t)stream, lds_launch, &c);
}

struct AtomCtx { float* acc; const int32_t* rows; int n, reps; };
static void atom_launch(hipStream_t s, void* c) {
  AtomCtx* x = (AtomCtx*)c;
  hipLaunchKernelGGL(atomic_rate_kernel, dim3(x->n), dim3(256), 0, s, x->acc, x->rows, x->reps);
}
float ceil_atomic(float* acc, const int32_t* rows, int n, int reps, void* stream) {
  AtomCtx c{acc, rows, n, reps};
  return timed((hipStream_t)stream, atom_launch, &c);
}

struct GatherCtx { int mode; const char* kv; const char* kr; const int32_t* idx; int blocks, nch; float* out; };
static void gather_launch(hipStream_t s, void* c) {
  GatherCtx* x = (GatherCtx*)c;
  hipLaunchKernelGGL(gather_rate_kernel, dim3(x->blocks), dim3(512), 0, s, x->mode, x->kv, x->kr, x->idx, x->nch, x->out);
}
float ceil_gather(int mode, const void* kv, const void* kr, const int32_t* idx, int blocks, int nch, float* out,
                  void* stream) {
  GatherCtx c{mode, (const char*)kv, (const char*)kr, idx, blocks, nch, out};
  return timed((hipStream_t)stream, gather_launch, &c);
}

}  // extern "C"
