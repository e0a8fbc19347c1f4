// Library-internal interface between the ABI sources: the scratch memory of
// the Spatial-Transformer block and the ResnetBlock2D handles, so that the
// U-Net, whose parts run one after another on one stream, gives all of them
// one arena instead of one workspace each.
#pragma once
#include <cstddef>
#include <utility>
#include <vector>

#include "../../include/st_block.h"
#include "../../include/st_resnet.h"

namespace stb {

// Device buffers of a handle whose contents do not outlive one forward
// (every byte a forward reads, the same forward wrote first): laid out back
// to back, 256-byte aligned, in one arena that is bound after create.
struct ScratchPlan {
  size_t bytes = 0;
  std::vector<std::pair<void**, size_t>> slots;
  // reserve n bytes for the pointer at *field (set by bind)
  template <typename T>
  void add(T** field, size_t n) {
    *field = nullptr;
    slots.push_back({reinterpret_cast<void**>(field), bytes});
    bytes += (n + 255) / 256 * 256;
  }
  // reserve n bytes and return their offset (for a caller that places the
  // buffer itself)
  size_t reserve(size_t n) {
    const size_t off = bytes;
    bytes += (n + 255) / 256 * 256;
    return off;
  }
  void bind(void* base) const {
    for (const auto& s : slots) *s.first = static_cast<char*>(base) + s.second;
  }
};

// Persistent device memory of several handles packed into one block.  The
// runtime rounds every allocation above 2 MB up to a multiple of 2 MB, which
// over the hundreds of weight matrices of a U-Net adds up to a large share
// of its memory.  A U-Net is therefore created twice: first with a counting
// arena (base == nullptr: every allocation still goes to hipMalloc, and its
// size, rounded to 256 bytes, is added to `counted`), then, after the first
// set of handles is destroyed, into one block of exactly that size
// (allocations in the same order, bump-allocated).
struct DevArena {
  char* base = nullptr;
  size_t cap = 0, used = 0, counted = 0;
  // nullptr with base set: the block is exhausted (an error)
  void* take(size_t n) {
    const size_t off = (used + 255) / 256 * 256;
    if (off + n > cap) return nullptr;
    used = off + n;
    return base + off;
  }
  void count(size_t n) { counted += (n + 255) / 256 * 256; }
};

}  // namespace stb

// Create with external scratch: the handle allocates its weights and the
// buffers that must outlive a forward, and leaves its scratch unbound; the
// caller gives it an arena of at least *_scratch_bytes() bytes (device
// memory of the same GPU, 256-byte aligned) with *_bind_scratch before the
// first forward, and keeps it for the handle's lifetime.  Handles bound to
// one arena must not run concurrently.  The public create calls bind an
// arena of their own.
// `persist` (may be NULL): the arena of the handle's persistent allocations
// (DevArena); the handle never frees memory taken from a block.
st_status stb_block_create(int B, int C, int H, int W, int heads, int D_ctx, int depth, st_dtype dtype,
                           const st_block_weights* w, void* stream, bool external_scratch,
                           stb::DevArena* persist, st_block** out);
size_t stb_block_scratch_bytes(const st_block* b);
void stb_block_bind_scratch(st_block* b, void* base);

st_status stb_resnet_create(int B, int Cin, int Cout, int H, int W, int Dt, float eps, st_dtype dtype,
                            const st_resnet_weights* w, void* stream, bool external_scratch,
                            stb::DevArena* persist, st_resnet** out);
size_t stb_resnet_scratch_bytes(const st_resnet* r);
void stb_resnet_bind_scratch(st_resnet* r, void* base);
