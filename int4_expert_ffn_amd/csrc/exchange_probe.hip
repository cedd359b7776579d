// Probe of the memory paths that the decode exchanges use, built into the
// profiling library only (-DFLINT_PHASE_TS): the XCD that each workgroup of a
// 256-workgroup launch runs on, and the round trip of one 32-bit value between
// two workgroups (stored by one, polled by the other, stored back, polled by
// the first) with the store and load cache policies of the exchanges.  Every
// poll loop is bounded; a pair that gives up reports no round trips.
#ifdef FLINT_PHASE_TS
#include <hip/hip_runtime.h>

#include <vector>

namespace flint {
namespace {

// XCC_ID hardware register (bits 3:0): the XCD the wave runs on.
__device__ __forceinline__ unsigned xcc_id() { return __builtin_amdgcn_s_getreg(20 | (0 << 6) | (3 << 11)); }

__global__ void k_probe_xcc(unsigned* out) {
  if (threadIdx.x == 0) out[blockIdx.x] = xcc_id();
}

constexpr int SC0 = 1, SC1 = 16;   // cache-policy bits of the buffer instructions

template <int LPOL>
__device__ __forceinline__ unsigned probe_load(unsigned* p) {
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(p, 0, 4, 0x00020000);
  return __builtin_amdgcn_raw_buffer_load_b32(rs, 0, 0, LPOL);
}

// SPOL < 0: the agent-scope atomic store of the exchanges; else a vector store
// with the given cache-policy bits
template <int SPOL>
__device__ __forceinline__ void probe_store(unsigned* p, unsigned v) {
  if constexpr (SPOL < 0) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(p, 0, 4, 0x00020000);
    __builtin_amdgcn_raw_buffer_store_b32(v, rs, 0, 0, SPOL);
  }
}

// Workgroups a and b exchange round r through f[0] (a -> b) and f[16] (b -> a);
// res[0] = rounds completed, res[1] = wall-clock ticks (100 MHz) for them.
template <int LPOL, int SPOL>
__global__ void k_probe_pingpong(unsigned* f, int a, int b, int rounds, long long* res) {
  if (threadIdx.x != 0) return;
  const int me = blockIdx.x;
  if (me != a && me != b) return;
  constexpr long long MAXPOLL = 2000000;
  const long long t0 = wall_clock64();
  int done = 0;
  for (int r = 1; r <= rounds; ++r) {
    long long k = 0;
    if (me == a) {
      probe_store<SPOL>(f, (unsigned)r);
      while (probe_load<LPOL>(f + 16) != (unsigned)r && ++k < MAXPOLL) asm volatile("" ::: "memory");
    } else {
      while (probe_load<LPOL>(f) != (unsigned)r && ++k < MAXPOLL) asm volatile("" ::: "memory");
      if (k < MAXPOLL) probe_store<SPOL>(f + 16, (unsigned)r);
    }
    if (k >= MAXPOLL) break;
    done = r;
  }
  if (me == a) {
    res[0] = done;
    res[1] = wall_clock64() - t0;
  }
}

}  // namespace

// xcc_of_block[256]: the XCD of each workgroup; round_trip_us[3]: round trip
// between workgroup 0 and another workgroup (agent-scope store, sc1 poll) on
// the same XCD and on another one, and (sc0 store, sc1 poll) on the same XCD;
// negative where the pair gave up.  Returns 0 or a HIP error code.
extern "C" int flint_moe_debug_exchange_probe(int* xcc_of_block, double* round_trip_us) {
  constexpr int NB = 256, ROUNDS = 2000;
  unsigned* ids = nullptr;
  unsigned* f = nullptr;
  long long* res = nullptr;
  hipError_t e = hipMalloc((void**)&ids, NB * 4);
  if (e == hipSuccess) e = hipMalloc((void**)&f, 4096);
  if (e == hipSuccess) e = hipMalloc((void**)&res, 64);
  std::vector<unsigned> h(NB, 0u);
  if (e == hipSuccess) {
    hipLaunchKernelGGL(k_probe_xcc, dim3(NB), dim3(64), 0, 0, ids);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipMemcpy(h.data(), ids, NB * 4, hipMemcpyDeviceToHost);
  int same = -1, other = -1;
  for (int i = 1; i < NB && e == hipSuccess; ++i) {
    if (same < 0 && h[i] == h[0]) same = i;
    if (other < 0 && h[i] != h[0]) other = i;
  }
  auto run = [&](auto kern, int b) -> double {
    if (e != hipSuccess || b < 0) return -1.0;
    long long r[2] = {0, 0};
    e = hipMemset(f, 0, 4096);
    if (e == hipSuccess) e = hipMemset(res, 0, 64);
    if (e == hipSuccess) {
      hipLaunchKernelGGL(kern, dim3(NB), dim3(64), 0, 0, f, 0, b, ROUNDS, res);
      e = hipGetLastError();
    }
    if (e == hipSuccess) e = hipMemcpy(r, res, 16, hipMemcpyDeviceToHost);
    return (e == hipSuccess && r[0] > 0) ? r[1] * 0.01 / r[0] : -1.0;
  };
  round_trip_us[0] = run(k_probe_pingpong<SC1, -1>, same);
  round_trip_us[1] = run(k_probe_pingpong<SC1, -1>, other);
  round_trip_us[2] = run(k_probe_pingpong<SC1, SC0>, same);
  for (int i = 0; i < NB; ++i) xcc_of_block[i] = (int)h[i];
  (void)hipFree(ids);
  (void)hipFree(f);
  (void)hipFree(res);
  return (int)e;
}

}  // namespace flint
#endif
