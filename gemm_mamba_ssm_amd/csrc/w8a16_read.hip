// Plain read of a device buffer: the HBM floor that the decode GEMV's weight
// stream is measured against. Every byte is read once with 16-byte buffer
// loads, non-temporal like the GEMV's weight loads; each lane issues all of
// its loads before it uses any, as the GEMV's one-group workgroups do, so the
// time is that of moving the bytes with the given launch shape and nothing
// else. The data are folded into one word per lane that is stored only under
// a condition the host never lets hold (bytes == 0 is a no-op there), so the
// compiler keeps the loads and the kernel writes nothing.
#include "w8a16_device.h"
#include "w8a16_host.h"

namespace w8a16 {
namespace {

constexpr uint32_t kReadFlags = 0x00020000;   // raw buffer, 32-bit data format
constexpr int kReadNonTemporal = 2;

template <int T, int L>
__global__ void __launch_bounds__(T) read_kernel(const uint8_t* __restrict__ p, uint32_t nbytes,
                                                 uint32_t* __restrict__ sink) {
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p), 0, nbytes, kReadFlags);
    const uint32_t base = blockIdx.x * static_cast<uint32_t>(T * L * 16) + threadIdx.x * 16u;
    u32x4_t v[L];
#pragma unroll
    for (int i = 0; i < L; ++i)      // offsets past nbytes read as zero
        v[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                               r, base + static_cast<uint32_t>(i * T * 16), 0, kReadNonTemporal));
    uint32_t x = 0;
#pragma unroll
    for (int i = 0; i < L; ++i) x ^= v[i][0] ^ v[i][1] ^ v[i][2] ^ v[i][3];
    if (nbytes == 0u && x == 1u) sink[threadIdx.x] = x;
}

template <int T>
int launch_read(const void* buf, int64_t bytes, int loads, void* sink, hipStream_t s) {
    const int64_t per_wg = static_cast<int64_t>(T) * loads * 16;
    const dim3 grid(static_cast<unsigned>(ceil_div(bytes, per_wg)));
    const uint8_t* p = static_cast<const uint8_t*>(buf);
    uint32_t* q = static_cast<uint32_t*>(sink);
    const uint32_t n = static_cast<uint32_t>(bytes);
    switch (loads) {
        case 1: return launch(&read_kernel<T, 1>, grid, dim3(T), s, p, n, q);
        case 2: return launch(&read_kernel<T, 2>, grid, dim3(T), s, p, n, q);
        case 4: return launch(&read_kernel<T, 4>, grid, dim3(T), s, p, n, q);
        case 8: return launch(&read_kernel<T, 8>, grid, dim3(T), s, p, n, q);
        default: return launch(&read_kernel<T, 16>, grid, dim3(T), s, p, n, q);
    }
}

}  // namespace
}  // namespace w8a16

extern "C" int w8a16_hbm_read(const void* buf, int64_t bytes, int threads, int loads, void* sink, void* stream) {
    using namespace w8a16;
    if (bytes < 0 || bytes % 16 != 0 || bytes > (int64_t{1} << 31)) return W8A16_ERR_SHAPE;
    if (threads != 64 && threads != 128 && threads != 256 && threads != 512 && threads != 1024) return W8A16_ERR_ARG;
    if (loads != 1 && loads != 2 && loads != 4 && loads != 8 && loads != 16) return W8A16_ERR_ARG;
    if (bytes == 0) return W8A16_OK;
    if (buf == nullptr || sink == nullptr) return W8A16_ERR_NULL;
    if (!aligned(buf, 16) || !aligned(sink, 4)) return W8A16_ERR_ALIGN;
    hipStream_t s = static_cast<hipStream_t>(stream);
    switch (threads) {
        case 64: return launch_read<64>(buf, bytes, loads, sink, s);
        case 128: return launch_read<128>(buf, bytes, loads, sink, s);
        case 256: return launch_read<256>(buf, bytes, loads, sink, s);
        case 512: return launch_read<512>(buf, bytes, loads, sink, s);
        default: return launch_read<1024>(buf, bytes, loads, sink, s);
    }
}
