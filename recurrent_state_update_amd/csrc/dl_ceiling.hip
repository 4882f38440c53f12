// dl_ceiling.hip -- a measurement helper beside libdeltalog, not part of the
// decode path: the step kernel's access pattern on the state with nothing
// else, so that the benchmark can report the HBM rate that pattern itself
// reaches on the GPU at hand next to the 8 TB/s peak.  Built into
// libdlceiling.so and loaded only by bench.py.
//
// One launch passes over a [BH, d_k, d_v] fp32 state in value tiles of
// T = min(d_v, 64) columns, one workgroup per (slot-head, tile), in the step
// kernel's block order and lane layout (4 adjacent columns per lane, rows
// strided by the workgroup), with its non-temporal loads:
//   write = 0  reads every tile once (the state traffic of an append step),
//              256 threads per tile;
//   write = 1  reads every tile and writes it back in place unchanged (the
//              state traffic of a merge step), 512 threads per tile where
//              the tile has that many 16-byte elements, as the merges take.
#include <hip/hip_runtime.h>

namespace {

using rsrc_t = __amdgpu_buffer_rsrc_t;
using u32x4 = unsigned int __attribute__((ext_vector_type(4)));

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, unsigned bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}

template <int DK, int DV, bool WRITE>
__global__ __launch_bounds__(WRITE ? 512 : 256) void tile_pass(float *S, float4 *sink, float key)
{
    constexpr int T = DV < 64 ? DV : 64;
    constexpr int THR = WRITE ? 512 : 256;
    constexpr int NT = DK * T / 4 < THR ? DK * T / 4 : THR;
    constexpr int LPR = T / 4, RPP = NT / LPR, P = DK / RPP, NTILE = DV / T;
    static_assert(P * RPP == DK && NT % 64 == 0, "tile shape");
    const int tid = threadIdx.x;
    const int sh = blockIdx.x / NTILE, tile = blockIdx.x % NTILE;
    const int c4 = tid % LPR, r0 = tid / LPR;
    const rsrc_t r = make_rsrc(S + (long)sh * DK * DV, DK * DV * 4);
    const unsigned off = (unsigned)(r0 * DV + tile * T + 4 * c4) * 4u;
    float4 x[P];
#pragma unroll
    for (int p = 0; p < P; ++p)
        x[p] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, off, p * RPP * DV * 4, 2));
    if (WRITE) {
#pragma unroll
        for (int p = 0; p < P; ++p)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x[p]), r, off, p * RPP * DV * 4, 0);
    } else {
        // keep the loads: a store that depends on every loaded value, taken
        // only if the sum equals `key` (the caller passes NaN: never)
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int p = 0; p < P; ++p) {
            acc.x += x[p].x;
            acc.y += x[p].y;
            acc.z += x[p].z;
            acc.w += x[p].w;
        }
        if (acc.x + acc.y + acc.z + acc.w == key)
            sink[(long)blockIdx.x * LPR + c4] = acc;
    }
}

template <int DK, int DV>
hipError_t launch(float *S, int BH, int write, float4 *sink, float key, hipStream_t st)
{
    constexpr int T = DV < 64 ? DV : 64;
    const dim3 grid((unsigned)BH * (DV / T));
    if (write) {
        constexpr int NT = DK * T / 4 < 512 ? DK * T / 4 : 512;
        hipLaunchKernelGGL((tile_pass<DK, DV, true>), grid, dim3(NT), 0, st, S, sink, key);
    } else {
        constexpr int NT = DK * T / 4 < 256 ? DK * T / 4 : 256;
        hipLaunchKernelGGL((tile_pass<DK, DV, false>), grid, dim3(NT), 0, st, S, sink, key);
    }
    return hipGetLastError();
}

} // namespace

extern "C" {

// Floats of sink a read pass may write: one float4 per lane column group of
// every workgroup (BH * d_v floats).  Returns 0 for an unsupported shape.
long dlc_sink_floats(int BH, int d_k, int d_v)
{
    if (BH <= 0 || !((d_k == 64 || d_k == 128) && (d_v == 64 || d_v == 128)))
        return 0;
    return (long)BH * d_v;
}

// One pass over the state S [BH, d_k, d_v] fp32 (16-byte aligned device
// memory) on `stream`: write = 0 reads it, write = 1 reads and rewrites it
// unchanged.  sink holds dlc_sink_floats() floats; key should be NaN, so that
// a read pass stores nothing.  d_k, d_v in {64, 128}.  Returns 0, or -1 for
// bad arguments, or the HIP error of the launch.
int dlc_tile_pass(float *S, int BH, int d_k, int d_v, int write, float *sink, float key, void *stream)
{
    if (!S || !sink || dlc_sink_floats(BH, d_k, d_v) == 0 || (long)BH * d_k * d_v >= (1L << 31) ||
        (reinterpret_cast<unsigned long>(S) & 15) || (reinterpret_cast<unsigned long>(sink) & 15))
        return -1;
    float4 *sk = reinterpret_cast<float4 *>(sink);
    const hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (d_k == 128 && d_v == 128)
        e = launch<128, 128>(S, BH, write, sk, key, st);
    else if (d_k == 128)
        e = launch<128, 64>(S, BH, write, sk, key, st);
    else if (d_v == 128)
        e = launch<64, 128>(S, BH, write, sk, key, st);
    else
        e = launch<64, 64>(S, BH, write, sk, key, st);
    return e == hipSuccess ? 0 : (int)e;
}

} // extern "C"
