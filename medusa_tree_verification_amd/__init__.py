"""MI355X-native Medusa verify step: heads + top-s, tree attention, acceptance."""
