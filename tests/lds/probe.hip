// lds/probe.hip -- LDS bank-conflict probe for gfx950 (test infrastructure,
// not part of the library).  One workgroup of 64 lanes repeats one LDS
// access 512 times; the 64 lane byte addresses (0xFFFFFFFF: lane inactive)
// and the access kind come from a table file, one dispatch per entry, so
// that rocprofv3's SQ_LDS_BANK_CONFLICT per dispatch divided by 512 is the
// conflict cycles of one access.  Every address is reduced into the 64 KiB
// array and aligned to the access size, so no access leaves it.
//
//   hipcc --offload-arch=gfx950 -O3 -std=c++17 tests/lds/probe.hip -o probe
//   probe <table>   (table: int32 n, then n x {int32 op, uint32 addr[64]};
//                    op 0..6 = read 16 B, read 8 B, read 4 B, transposing
//                    read 8 B, write 16 B, write 8 B, write 4 B)
#include <hip/hip_runtime.h>
#include <cstdio>
#include <cstdint>
#include <vector>
typedef short s4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));
enum { RD128 = 0, RD64 = 1, RD32 = 2, RDTR = 3, WR128 = 4, WR64 = 5, WR32 = 6 };
constexpr int kLds = 65536;
constexpr int kReps = 512;

template <int OP>
__global__ void __launch_bounds__(64) probe(const uint32_t* addr, uint32_t* sink) {
  __shared__ __align__(16) unsigned char lds[kLds];
  const int l = threadIdx.x;
  for (int i = l; i < kLds / 16; i += 64) reinterpret_cast<uint4*>(lds)[i] = uint4{(uint32_t)i, 1u, 2u, 3u};
  __syncthreads();
  constexpr uint32_t w = (OP == RD128 || OP == WR128) ? 16 : (OP == RD32 || OP == WR32) ? 4 : 8;
  const bool on = addr[l] != 0xFFFFFFFFu;
  uint32_t a = addr[l] % (kLds - 16);
  a &= ~(w - 1);
  uint32_t acc = 0;
  for (int r = 0; r < kReps; ++r) {
    asm volatile("" : "+v"(a));
    if (!on) continue;
    if constexpr (OP == RD128) { u4 v = *((volatile __attribute__((address_space(3))) u4*)(lds + a)); acc ^= v[0] ^ v[3]; }
    if constexpr (OP == RD64) { u2 v = *((volatile __attribute__((address_space(3))) u2*)(lds + a)); acc ^= v[0] ^ v[1]; }
    if constexpr (OP == RD32) { acc ^= *((volatile __attribute__((address_space(3))) uint32_t*)(lds + a)); }
    if constexpr (OP == RDTR) {
      s4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4*)(lds + a));
      acc ^= (uint32_t)(uint16_t)v[0] ^ ((uint32_t)(uint16_t)v[3] << 16);
    }
    if constexpr (OP == WR128) *((volatile __attribute__((address_space(3))) u4*)(lds + a)) = u4{acc, 1u, 2u, (uint32_t)r};
    if constexpr (OP == WR64) *((volatile __attribute__((address_space(3))) u2*)(lds + a)) = u2{acc, (uint32_t)r};
    if constexpr (OP == WR32) *((volatile __attribute__((address_space(3))) uint32_t*)(lds + a)) = acc + r;
  }
  __syncthreads();
  sink[l] = acc ^ reinterpret_cast<uint32_t*>(lds)[l];
}

int main(int argc, char** argv) {
  const char* path = argc > 1 ? argv[1] : "patterns.bin";
  FILE* f = fopen(path, "rb");
  if (!f) { fprintf(stderr, "no %s\n", path); return 1; }
  int n = 0;
  if (fread(&n, 4, 1, f) != 1 || n <= 0 || n > 100000) return 1;
  std::vector<int> ops(n);
  std::vector<uint32_t> tab(static_cast<size_t>(n) * 64);
  for (int i = 0; i < n; ++i) {
    if (fread(&ops[i], 4, 1, f) != 1 || fread(&tab[i * 64], 4, 64, f) != 64) return 1;
    if (ops[i] < 0 || ops[i] > 6) return 1;
  }
  fclose(f);
  uint32_t *d_addr, *d_sink;
  if (hipMalloc(&d_addr, tab.size() * 4) != hipSuccess) return 1;
  if (hipMalloc(&d_sink, 64 * 4) != hipSuccess) return 1;
  if (hipMemcpy(d_addr, tab.data(), tab.size() * 4, hipMemcpyHostToDevice) != hipSuccess) return 1;
  for (int i = 0; i < n; ++i) {
    const uint32_t* p = d_addr + static_cast<size_t>(i) * 64;
    switch (ops[i]) {
      case RD128: probe<RD128><<<1, 64>>>(p, d_sink); break;
      case RD64: probe<RD64><<<1, 64>>>(p, d_sink); break;
      case RD32: probe<RD32><<<1, 64>>>(p, d_sink); break;
      case RDTR: probe<RDTR><<<1, 64>>>(p, d_sink); break;
      case WR128: probe<WR128><<<1, 64>>>(p, d_sink); break;
      case WR64: probe<WR64><<<1, 64>>>(p, d_sink); break;
      case WR32: probe<WR32><<<1, 64>>>(p, d_sink); break;
    }
    if (hipDeviceSynchronize() != hipSuccess) { fprintf(stderr, "failed at %d\n", i); return 1; }
  }
  printf("probe: %d patterns done\n", n);
  return 0;
}
