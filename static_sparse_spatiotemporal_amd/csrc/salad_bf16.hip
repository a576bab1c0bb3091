// SALAD gate and output (SALAD page, sections 2.1-2.2): the scalar gate of
// the linear branch and the gated, projected sum of the two branches.
//
//   k_salad_gate_part   per (sample, part of its tokens): the sum over the
//                       part's tokens of sigmoid(x . w + bias); one wave per
//                       token (16 bytes per lane per load), w staged in LDS;
//   k_salad_gate_final  per sample: the parts summed in a fixed order / N
//                       (deterministic);
//   k_salad_combine<D>  out = O_s + g[b] (O_l W^T + bias) over the
//                       merged-head channels c = h D + e.  One workgroup
//                       (8 waves) computes a 256-token x 256-channel tile of
//                       the product as C^T = W A^T with 32x32x16 bf16 MFMAs:
//                       64-channel K steps copied HBM -> LDS with
//                       global_load_lds into double buffers (one LDS array
//                       each), operands read with ds_read_b128 from
//                       XOR-swizzled rows.  Each wave then stages its fp32
//                       result in LDS and reads O_s and writes out in
//                       256-byte row pieces.
#include <mutex>

#include "attn_common.h"
#include "salad.h"

namespace tra {
namespace {

#define LDS_AS __attribute__((address_space(3)))

// ---------------------------------------------------------------- gate ----

constexpr int kGateThreads = 256;
constexpr int kGateRows = 64;       // tokens per part (at least)
constexpr int kGateMaxParts = 1024;

int gate_parts(int64_t N)
{
    const int64_t p = (N + kGateRows - 1) / kGateRows;
    return (int)(p < 1 ? 1 : p > kGateMaxParts ? kGateMaxParts : p);
}

struct GateArgs {
    const __bf16 *x;
    int64_t sxb, sxn;  // element strides of sample and token
    const __bf16 *w;
    float bias;
    int32_t B, C, parts;
    int64_t N, rows_per_part;
    float *part;  // [B][parts]
    float *gate;  // [B]
};

__global__ __launch_bounds__(kGateThreads) void k_salad_gate_part(GateArgs a)
{
    // w stays bf16 in LDS: a lane's 8 values are then 16 contiguous bytes
    // (one ds_read_b128, 16 lanes covering the 64 banks once), and each
    // pair of products goes through one bf16 dot instruction (products of
    // bf16 values are exact in fp32).
    extern __shared__ __attribute__((aligned(16))) __bf16 sW[];  // C values
    __shared__ float sSum[kGateThreads / 64];
    const int b = blockIdx.y, part = blockIdx.x;
    for (int c = threadIdx.x; c < a.C; c += kGateThreads)
        sW[c] = a.w[c];
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t n0 = (int64_t)part * a.rows_per_part;
    const int64_t n1 = n0 + a.rows_per_part < a.N ? n0 + a.rows_per_part : a.N;
    float acc = 0.f;
    for (int64_t n = n0 + wave; n < n1; n += kGateThreads / 64) {
        const __bf16 *row = a.x + b * a.sxb + n * a.sxn;
        float z = 0.f;
        for (int c = lane * 8; c < a.C; c += 512) {
            const uint4 v = *(const uint4 *)(row + c);
            const uint4 wv = *(const uint4 *)(sW + c);
            const uint32_t vs[4] = {v.x, v.y, v.z, v.w}, ws[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
            for (int j = 0; j < 4; ++j)
                z = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, vs[j]), __builtin_bit_cast(bf16x2, ws[j]),
                                                    z, false);
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1)
            z += __shfl_xor(z, off);
        acc += 1.f / (1.f + __expf(-(z + a.bias)));
    }
    if (lane == 0)
        sSum[wave] = acc;
    __syncthreads();
    if (threadIdx.x == 0)
        a.part[(int64_t)b * a.parts + part] = (sSum[0] + sSum[1]) + (sSum[2] + sSum[3]);
}

// One wave per sample: lane l sums parts l, l + 64, ..., then a butterfly;
// lane 0's result is the same on every run.
__global__ __launch_bounds__(64) void k_salad_gate_final(GateArgs a)
{
    const int b = blockIdx.x, lane = threadIdx.x;
    float s = 0.f;
    for (int p = lane; p < a.parts; p += 64)
        s += a.part[(int64_t)b * a.parts + p];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        s += __shfl_xor(s, off);
    if (lane == 0)
        a.gate[b] = s / (float)a.N;
}

// ------------------------------------------------------------- combine ----

// Wave layouts of a 256 x 256 tile: NW = 8 waves of 64 tokens x 128
// channels (4 x 2, two waves per SIMD), or NW = 4 waves of 128 x 128 (2 x 2,
// one wave per SIMD, 256 accumulator registers).
template <int NW>
struct CGeo {
    static constexpr int THREADS = 64 * NW;
    static constexpr int WM = NW == 8 ? 4 : 2;    // waves along tokens
    static constexpr int TMW = 256 / WM;          // tokens per wave
    static constexpr int TT = TMW / 32;           // 32-token MFMA tiles per wave
    static constexpr int CT = 4;                  // 32-channel MFMA tiles per wave (128 channels)
    static constexpr int NCP = 32 / NW;           // 1 KB copy instructions per operand per wave
};
constexpr int kTM = 256;             // tokens per tile
constexpr int kTN = 256;             // output channels per tile
constexpr int kTK = 64;              // input channels per K step
constexpr int kRowB = kTK * 2;       // bytes per LDS tile row
constexpr int kTileB = 256 * kRowB;  // 32 KB per operand tile
// The 4-wave layout halves the operand bytes read from LDS per MFMA, but
// with 256 accumulators per wave the compiler spills (87 registers); the
// 8-wave layout is the one launched.
constexpr int kCombineWaves = 8;
constexpr int kGroupM = 8;           // token tiles per group of the tile order
constexpr int kXcds = 8;

struct CombineArgs {
    const __bf16 *os, *ol;
    __bf16 *out;
    int64_t s_os[3], s_ol[3], s_out[3];
    const __bf16 *w;     // [C][C]
    const float *bias;   // [C] or null
    const float *gate;   // [B]
    int64_t N, M;        // tokens per sample, B * N
    int32_t C, mt, nt, tiles, per_xcd;
};

// Physical 16-byte chunk of logical chunk c in LDS row `row` (8 per row).
// A 128-byte row is half of the 64 banks, so rows r and r + 1 share a bank
// line; the 16 rows of one ds_read_b128 pass then need distinct chunks
// within each row parity, which (r >> 1) & 7 gives (r & 7 repeats at r + 8:
// 2-way conflicts).
__device__ inline int cswz(int row) { return (row >> 1) & 7; }

__device__ inline void wait_copies() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <int D, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(8 / NW, 8 / NW)))
void k_salad_combine(CombineArgs a)
{
    using G = CGeo<NW>;
    // double buffers, one LDS array each (see the attention forward kernel:
    // statically named buffers keep the copy into one from delaying the
    // reads of the other)
    __shared__ __attribute__((aligned(1024))) char sA0[kTileB];
    __shared__ __attribute__((aligned(1024))) char sA1[kTileB];
    __shared__ __attribute__((aligned(1024))) char sW0[kTileB];
    __shared__ __attribute__((aligned(1024))) char sW1[kTileB];

    // tile order: XCD x takes tiles [x per_xcd, (x + 1) per_xcd) of the
    // grouped order (kGroupM token tiles x all channel tiles, token tile
    // fastest), so the workgroups resident on one XCD share A and W slices
    // in its L2
    const int t = (blockIdx.x % kXcds) * a.per_xcd + blockIdx.x / kXcds;
    if (t >= a.tiles)
        return;
    const int gsize = kGroupM * a.nt;
    const int g = t / gsize, r = t - g * gsize;
    const int gm = a.mt - g * kGroupM < kGroupM ? a.mt - g * kGroupM : kGroupM;
    const int mtile = g * kGroupM + r % gm, ntile = r / gm;
    const int64_t m0 = (int64_t)mtile * kTM;
    const int n0 = ntile * kTN;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave % G::WM, wn = wave / G::WM;
    const int l32 = lane & 31, hh = lane >> 5;
    const int C = a.C;
    const int nsteps = C / kTK;

    // Copy geometry: copy instruction i of wave w fills LDS bytes
    // (NW i + w) KB .. of a tile, i.e. rows 8 (NW i + w) + lane / 8; lane
    // position p = lane % 8 receives logical chunk p ^ cswz(row).
    int64_t aoff[G::NCP];  // element offset of the token row of copy i (no channel part)
    int64_t woff[G::NCP];  // element offset of the weight row of copy i plus the chunk
    int achunk[G::NCP];
#pragma unroll
    for (int i = 0; i < G::NCP; ++i) {
        const int row = 8 * (NW * i + wave) + lane / 8;
        const int c = (lane % 8) ^ cswz(row);
        uint32_t R = (uint32_t)(m0 + row);
        R = R < (uint32_t)a.M ? R : (uint32_t)a.M - 1u;
        const uint32_t bb = R / (uint32_t)a.N, nn = R - bb * (uint32_t)a.N;  // B N < 2^31
        aoff[i] = (int64_t)bb * a.s_ol[0] + (int64_t)nn * a.s_ol[2];
        achunk[i] = 8 * c;
        int co = n0 + row;
        co = co < C ? co : C - 1;
        woff[i] = (int64_t)co * C + 8 * c;
    }
    auto copy_step = [&](int step, char LDS_AS *dA, char LDS_AS *dW) {
        const int k0 = step * kTK;
        const int h = k0 / D, e0 = k0 - h * D;  // a 64-channel step lies inside one head
        const __bf16 *ap = a.ol + h * a.s_ol[1] + e0;
        const __bf16 *wp = a.w + k0;
#pragma unroll
        for (int i = 0; i < G::NCP; ++i) {
            __builtin_amdgcn_global_load_lds((const void *)(ap + aoff[i] + achunk[i]),
                                             (void LDS_AS *)(dA + (NW * i + wave) * 1024), 16, 0, 0);
            __builtin_amdgcn_global_load_lds((const void *)(wp + woff[i]),
                                             (void LDS_AS *)(dW + (NW * i + wave) * 1024), 16, 0, 0);
        }
    };

    // Fragment offsets (bytes inside a tile) for k-substep ks of a K step:
    // W rows wn 128 + ct 32 + lane % 32 (A operand of C^T = W A^T), token
    // rows wm 64 + tt 32 + lane % 32 (B operand), chunk 2 ks + lane / 32.
    auto frag = [&](int row, int ks) { return row * kRowB + (((2 * ks + hh) ^ cswz(row)) << 4); };

    f32x16 acc[G::CT][G::TT];
#pragma unroll
    for (int ct = 0; ct < G::CT; ++ct)
#pragma unroll
        for (int tt = 0; tt < G::TT; ++tt)
            acc[ct][tt] = f32x16{};

    copy_step(0, (char LDS_AS *)sA0, (char LDS_AS *)sW0);
    for (int s2 = 0; s2 < nsteps; s2 += 2)
#pragma unroll
    for (int buf = 0; buf < 2; ++buf) {
        const int step = s2 + buf;
        if (step >= nsteps)
            break;
        // step's copies have landed everywhere and every wave is done with
        // the previous step, whose buffers receive the next step (the last
        // step re-copies itself so that every path issues the same copies)
        wait_copies();
        __syncthreads();
        copy_step(step + 1 < nsteps ? step + 1 : step, (char LDS_AS *)(buf == 0 ? sA1 : sA0),
                  (char LDS_AS *)(buf == 0 ? sW1 : sW0));
        // the copies go out before the step's MFMAs (left to itself the
        // scheduler sinks them to the end of the step, and the next step's
        // wait then exposes their whole latency)
        __builtin_amdgcn_sched_barrier(0);
        const char LDS_AS *tA = (const char LDS_AS *)(buf == 0 ? sA0 : sA1);
        const char LDS_AS *tW = (const char LDS_AS *)(buf == 0 ? sW0 : sW1);
        // fragments of k-substep ks + 1 are read while those of ks feed the
        // MFMAs
        bf16x8 wf[2][G::CT], af[2][G::TT];
        auto read_frags = [&](int ks, int x) {
#pragma unroll
            for (int ct = 0; ct < G::CT; ++ct)
                wf[x][ct] = *(const bf16x8 LDS_AS *)(tW + frag(wn * 128 + ct * 32 + l32, ks));
#pragma unroll
            for (int tt = 0; tt < G::TT; ++tt)
                af[x][tt] = *(const bf16x8 LDS_AS *)(tA + frag(wm * G::TMW + tt * 32 + l32, ks));
        };
        read_frags(0, 0);
#pragma unroll
        for (int ks = 0; ks < kTK / 16; ++ks) {
            __builtin_amdgcn_sched_barrier(0);
            if (ks + 1 < kTK / 16)
                read_frags(ks + 1, (ks + 1) & 1);
#pragma unroll
            for (int ct = 0; ct < G::CT; ++ct)
#pragma unroll
                for (int tt = 0; tt < G::TT; ++tt)
                    acc[ct][tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[ks & 1][ct], af[ks & 1][tt],
                                                                          acc[ct][tt], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    wait_copies();
    __syncthreads();  // every wave is done with the operand tiles

    // Epilogue.  acc[ct][tt] lane holds C^T[channel wn 128 + ct 32 + 8 (i / 4)
    // + 4 hh + i % 4][token wm 64 + tt 32 + lane % 32].  Per token tile tt the
    // wave writes its 32 tokens x 128 channels (fp32, 512-byte rows, 16-byte
    // chunks XOR-swizzled by row) into 16 KB of its own, then reads them back
    // 4 channels per lane, a whole 128-channel row per half-wave.
    // (16 KB per wave: the 128 KB of operand tiles hold 8 such regions)
    char LDS_AS *st = (char LDS_AS *)(wave < 2 ? sA0 : wave < 4 ? sA1 : wave < 6 ? sW0 : sW1) + (wave & 1) * 16384;
#pragma unroll
    for (int tt = 0; tt < G::TT; ++tt) {
#pragma unroll
        for (int ct = 0; ct < G::CT; ++ct)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                f32x4 v;
#pragma unroll
                for (int x = 0; x < 4; ++x)
                    v[x] = acc[ct][tt][4 * q + x];
                const int ch = (8 * ct + 2 * q + hh) ^ (l32 & 31);
                *(f32x4 LDS_AS *)(st + l32 * 512 + ch * 16) = v;
            }
        const int chunk = lane & 31;
        const int cglob = n0 + wn * 128 + 4 * chunk;
        const bool col_ok = cglob < C;
        const int hp = cglob / D, ep = cglob - hp * D;
        f32x4 bias4 = {0.f, 0.f, 0.f, 0.f};
        if (a.bias != nullptr && col_ok)
            bias4 = *(const f32x4 *)(a.bias + cglob);
        // The O_s pieces and gate values of all 16 rows are loaded before
        // any is used (addresses clamped into the tensors, stores masked),
        // so that their latencies overlap instead of adding up row by row.
        const int hpc = col_ok ? hp : 0, epc = col_ok ? ep : 0;
        bf16x4 o4[16];
        float gv[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            uint32_t R = (uint32_t)(m0 + wm * G::TMW + tt * 32 + 2 * i + hh);
            R = R < (uint32_t)a.M ? R : (uint32_t)a.M - 1u;
            const uint32_t bb = R / (uint32_t)a.N, nn = R - bb * (uint32_t)a.N;
            gv[i] = a.gate[bb];
            o4[i] = *(const bf16x4 *)(a.os + (int64_t)bb * a.s_os[0] + hpc * a.s_os[1] + (int64_t)nn * a.s_os[2] +
                                      epc);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int row = 2 * i + hh;
            const f32x4 v = *(const f32x4 LDS_AS *)(st + row * 512 + ((chunk ^ (row & 31)) << 4));
            const uint32_t R = (uint32_t)(m0 + wm * G::TMW + tt * 32 + row);
            f32x4 res;
#pragma unroll
            for (int x = 0; x < 4; ++x)
                res[x] = (float)o4[i][x] + gv[i] * (v[x] + bias4[x]);
            if (R < (uint32_t)a.M && col_ok) {
                const uint32_t bb = R / (uint32_t)a.N, nn = R - bb * (uint32_t)a.N;
                *(bf16x4 *)(a.out + (int64_t)bb * a.s_out[0] + hp * a.s_out[1] + (int64_t)nn * a.s_out[2] + ep) =
                    __builtin_convertvector(res, bf16x4);
            }
        }
    }
}

}  // namespace

size_t salad_gate_workspace_bytes(int64_t B, int64_t N)
{
    const size_t bytes = (size_t)B * gate_parts(N) * sizeof(float);
    return (bytes + 255) / 256 * 256;
}

hipError_t launch_salad_gate(const void *x, const int64_t sx[2], const void *w, float bias, int64_t B, int64_t N,
                             int64_t C, float *gate, void *workspace, hipStream_t stream)
{
    GateArgs a{};
    a.x = (const __bf16 *)x;
    a.sxb = sx[0];
    a.sxn = sx[1];
    a.w = (const __bf16 *)w;
    a.bias = bias;
    a.B = (int32_t)B;
    a.C = (int32_t)C;
    a.parts = gate_parts(N);
    a.N = N;
    a.rows_per_part = (N + a.parts - 1) / a.parts;
    a.part = (float *)workspace;
    a.gate = gate;
    hipLaunchKernelGGL(k_salad_gate_part, dim3((unsigned)a.parts, (unsigned)B), dim3(kGateThreads),
                       (size_t)C * sizeof(__bf16), stream, a);
    hipLaunchKernelGGL(k_salad_gate_final, dim3((unsigned)B), dim3(64), 0, stream, a);
    return hipGetLastError();
}

// ------------------------------------------ gate without allocation ----

// The gate's partial sums in a fixed device array, for callers that cannot
// allocate or bring a workspace (code under graph capture, serving loops).
// Each device holds its own copy until the process ends.  In host code the
// name `scratch` is only a host-side stand-in: the device address comes from
// hipGetSymbolAddress, once per device with that device current, and only
// that address is ever passed to a kernel.
static __device__ __align__(256) float scratch[kGateScratchFloats];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices] = {};
}  // namespace

bool salad_gate_scratch_fits(int64_t B, int64_t N)
{
    return B >= 0 && (int64_t)gate_parts(N) * B <= kGateScratchFloats;
}

hipError_t launch_salad_gate_scratch(const void *x, const int64_t sx[2], const void *w, float bias, int64_t B,
                                     int64_t N, int64_t C, float *gate, hipStream_t stream)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    void *ptr = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        if (g_scratch[dev] == nullptr) {
            e = hipGetSymbolAddress(&g_scratch[dev], HIP_SYMBOL(scratch));
            if (e != hipSuccess) {
                g_scratch[dev] = nullptr;
                return e;
            }
        }
        ptr = g_scratch[dev];
    }
    // every (sample, part) slot is written by the part kernel before the
    // final kernel reads it, so the array needs no clearing between calls
    return launch_salad_gate(x, sx, w, bias, B, N, C, gate, ptr, stream);
}

hipError_t launch_salad_combine(const void *os, const int64_t s_os[3], const void *ol, const int64_t s_ol[3],
                                void *out, const int64_t s_out[3], const void *w, const float *bias,
                                const float *gate, int64_t B, int64_t H, int64_t N, int64_t D, hipStream_t stream)
{
    CombineArgs a{};
    a.os = (const __bf16 *)os;
    a.ol = (const __bf16 *)ol;
    a.out = (__bf16 *)out;
    for (int j = 0; j < 3; ++j) {
        a.s_os[j] = s_os[j];
        a.s_ol[j] = s_ol[j];
        a.s_out[j] = s_out[j];
    }
    a.w = (const __bf16 *)w;
    a.bias = bias;
    a.gate = gate;
    a.N = N;
    a.M = B * N;
    a.C = (int32_t)(H * D);
    a.mt = (int32_t)((a.M + kTM - 1) / kTM);
    a.nt = (a.C + kTN - 1) / kTN;
    a.tiles = a.mt * a.nt;
    a.per_xcd = (a.tiles + kXcds - 1) / kXcds;
    const dim3 grid((unsigned)(a.per_xcd * kXcds));
    constexpr int NW = kCombineWaves;
    if (D == 128)
        hipLaunchKernelGGL((k_salad_combine<128, NW>), grid, dim3(64 * NW), 0, stream, a);
    else
        hipLaunchKernelGGL((k_salad_combine<64, NW>), grid, dim3(64 * NW), 0, stream, a);
    return hipGetLastError();
}

}  // namespace tra
