// ll_packet.hpp -- the LL protocol's flagged packets, device side.
#pragma once

#include "ar_device.hpp"

namespace ar {

// Packet word of the LL protocol: low 32 bits payload, high 32 bits flag.
// Written and read as one aligned 64-bit access at agent (device) scope, so
// payload and flag become visible together to a reader on any XCD.
__device__ inline void put_packet(uint64_t *slot, uint32_t payload, uint32_t flag)
{
    __hip_atomic_store(slot, ((uint64_t)flag << 32) | payload, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline uint64_t read_packet(const uint64_t *slot)
{
    return __hip_atomic_load(const_cast<uint64_t *>(slot), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline uint32_t packet_flag(uint64_t pkt) { return (uint32_t)(pkt >> 32); }
__device__ inline uint32_t packet_payload(uint64_t pkt) { return (uint32_t)pkt; }

// Packet access by width.  PW payload words per packet, each word next to its
// own flag: PW = 1 is the 8-byte packet {payload, flag}; PW = 2 the 16-byte
// packet {payload0, flag, payload1, flag}.  A reader accepts a 16-byte
// packet only when both flags are set, so it needs each 8-byte half to be
// written as a unit: the 8-byte packet has that from its 64-bit atomic store,
// the 16-byte one only from the hardware (see below).  The 16-byte packet
// halves the memory instructions per payload byte.
// Indices count packets of the width from the packet region's base.
template <int PW>
struct PacketIO;

template <>
struct PacketIO<1> {
    using V = uint64_t;
    uint64_t *base;
    __device__ PacketIO(uint64_t *pkts, uint64_t) : base(pkts) {}
    __device__ V load(uint64_t i) const { return read_packet(base + i); }
    __device__ void store(uint64_t i, const uint32_t *w, uint32_t flag) const
    {
        put_packet(base + i, w[0], flag);
    }
    __device__ void clear(uint64_t i) const { put_packet(base + i, 0u, 0u); }
    __device__ static bool ready(V v, uint32_t want) { return packet_flag(v) == want; }
    __device__ static uint32_t word(V v, int) { return packet_payload(v); }
};

// 16-byte packets go through buffer instructions: one 128-bit load or store
// with the same coherence bit (sc1) that the 64-bit agent-scope atomics above
// compile to on gfx950, and with the packet region as the buffer's extent, so
// an index past the region cannot touch other memory (reads give 0, writes
// are dropped).  The region must stay below 4 GiB (32-bit byte offsets).
//
// Unlike the 8-byte packet, this width rests on a property no document
// grants: HIP offers no 128-bit atomic, and nothing in the gfx950 ISA or the
// AMDGPU memory model says that each 8-byte half of a 128-bit store becomes
// visible as a unit.  A half that tore could show a set flag beside a stale
// payload.  So the 16-byte packet is an ablation that a caller must ask for
// (arOptLLPacketBytes = 16); the defaults and the tuner use 8-byte packets,
// whose {payload, flag} pair is one 64-bit atomic store.
template <>
struct PacketIO<2> {
    using V = u32x4;
    static constexpr int kCoherent = 16;             // cache-policy bit sc1
    // Poll loads also carry the compiler's volatile bit (aux bit 31), so a
    // re-read inside the wait loop can never be merged with an earlier one.
    static constexpr int kPoll = kCoherent | (int)0x80000000u;
    static constexpr int kRawBufferWord3 = 0x00020000; // gfx9 raw buffer descriptor
    __amdgpu_buffer_rsrc_t rsrc;
    __device__ PacketIO(uint64_t *pkts, uint64_t region_bytes)
        : rsrc(__builtin_amdgcn_make_buffer_rsrc(pkts, 0, (int)(uint32_t)region_bytes,
                                                 kRawBufferWord3))
    {
    }
    __device__ V load(uint64_t i) const
    {
        return __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)(uint32_t)(i * 16u), 0, kPoll);
    }
    __device__ void store(uint64_t i, const uint32_t *w, uint32_t flag) const
    {
        const V v = {w[0], flag, w[1], flag};
        __builtin_amdgcn_raw_buffer_store_b128(v, rsrc, (int)(uint32_t)(i * 16u), 0, kCoherent);
    }
    __device__ void clear(uint64_t i) const
    {
        const V z = {0u, 0u, 0u, 0u};
        __builtin_amdgcn_raw_buffer_store_b128(z, rsrc, (int)(uint32_t)(i * 16u), 0, kCoherent);
    }
    __device__ static bool ready(V v, uint32_t want) { return v.y == want && v.w == want; }
    __device__ static uint32_t word(V v, int e) { return e == 0 ? v.x : v.z; }
};

}  // namespace ar
