// The warm tier's state and limits as the launches carry them (plain data).
#pragma once

#include <stdint.h>

namespace hga {

constexpr int kWarmMaxSlots = 1024;
constexpr int kWarmMaxList = 256;     // top_g limit with the warm tier
constexpr int kWarmMapGroups = 8192;  // contexts of up to this many groups per (b, kv head) use the LDS map

// The caller's LRU state and this step's outputs (device memory).
struct WarmState {
  int32_t* tags;      // [B*Hkv, slots] group of each slot, -1 empty
  int32_t* stamps;    // [B*Hkv, slots] last step that used each slot
  int32_t* clock;     // [B*Hkv] steps taken
  int32_t* hits;      // nullable [B*Hkv]
  int32_t* misses;    // nullable [B*Hkv]
  int32_t* slot_of;   // ws [B*Hkv, top_g]: the slot list
  int32_t slots;
};

}  // namespace hga
